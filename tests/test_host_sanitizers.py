"""Host AddressSanitizer / UndefinedBehaviorSanitizer runs (no GPU needed).

* The CPU oracle (oracle/moe_oracle.c) built with gcc and both sanitizers,
  driven by tests/sanitize/oracle_driver.c: every exported oracle function on
  small random banks of every codec, its invalid-argument paths, and the
  agreement of its per-pair, union and single-element evaluations.
* The library sources built with the sanitizers on their host side (device
  code at -O0: it is never launched here) and linked into
  tests/sanitize/abi_host_driver.cpp, which runs the C ABI's host-side error
  paths, path selection and workspace sizes, and the allocation-free entry
  point's scratch check -- all of which return before any HIP runtime call.

Any sanitizer report makes the driver exit non-zero (no recovery).  Leak
checking is off: the HIP runtime's own start-up allocations are not this
library's.
"""

import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "quantized_expert_gather_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, cwd, env=None, timeout=600):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=env, timeout=timeout)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_oracle_under_asan_ubsan():
    with tempfile.TemporaryDirectory(prefix="orc_san_") as tmp:
        exe = os.path.join(tmp, "oracle_san")
        rc, out = _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall", "-Wextra",
                        os.path.join(ROOT, "oracle", "moe_oracle.c"), os.path.join(SAN, "oracle_driver.c"),
                        "-lm", "-o", exe], tmp)
        assert rc == 0, out
        rc, out = _run([exe], tmp, ENV)
        print(out)
        assert rc == 0, out
        assert "all checks passed" in out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm compilers missing")
def test_abi_host_validation_under_asan_ubsan():
    host_san = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                "-Xarch_host", "-fno-omit-frame-pointer"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with tempfile.TemporaryDirectory(prefix="abi_san_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            rc, out = _run([HIPCC, "--offload-arch=gfx950", "-O1", "-Xarch_device", "-O0", "-std=c++17", "-fPIC",
                            *host_san, *inc, "-c", src, "-o", obj], tmp)
            return obj, rc, out

        with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
            results = list(ex.map(compile_one, srcs))
        for obj, rc, out in results:
            assert rc == 0, out
        drv = os.path.join(tmp, "driver.o")
        rc, out = _run([HIPCC, "-O1", "-g", "-std=c++17", *host_san, "-I", os.path.join(ROOT, "include"), "-c",
                        os.path.join(SAN, "abi_host_driver.cpp"), "-o", drv], tmp)
        assert rc == 0, out
        exe = os.path.join(tmp, "abi_san")
        rc, out = _run([CLANGXX, "-fsanitize=address,undefined", *[r[0] for r in results], drv,
                        "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe], tmp)
        assert rc == 0, out
        rc, out = _run([exe], tmp, ENV)
        print(out)
        assert rc == 0, out
        assert "all checks passed" in out
