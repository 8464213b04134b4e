"""Builds libmoe_q4.so (HIP, gfx950) in-tree with hipcc.

Each source compiles to its own object in parallel (the kernel template
instantiations are split over several units), then one link step makes the
shared library.
"""

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_q4.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU forms stay off: plain scalar / float2 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _filter(text: str) -> str:
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False, extra=(), jobs: int = 0) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, os.cpu_count() or 1), 16)
    with tempfile.TemporaryDirectory(prefix="moe_q4_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [hipcc, *HIPCC_FLAGS, *extra, *inc, "-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            return src, obj, r.returncode, _filter(r.stdout + r.stderr), cmd

        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(compile_one, srcs))
        for src, obj, rc, out, cmd in results:
            if verbose:
                print(" ".join(cmd), flush=True)
                if out.strip():
                    print(out, flush=True)
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {os.path.basename(src)} ({rc}):\n{out}")
        tmp_lib = LIB + ".tmp"
        link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *[r[1] for r in results], "-o", tmp_lib]
        r = subprocess.run(link, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed ({r.returncode}):\n{_filter(r.stdout + r.stderr)}")
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, extra=[a for a in sys.argv[1:] if a != "-v"])
