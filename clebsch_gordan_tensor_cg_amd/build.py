"""Build the cgtp HIP library for gfx950 in-tree (no GPU needed).

    python -m clebsch_gordan_tensor_cg_amd.build [--aot]

Compiles csrc/*.cpp and csrc/*.hip with hipcc into libcgtp.so next to this
file.  With --aot, also plans the standard workloads with
CGTP_PLAN_NO_LOAD so their generated kernels are compiled into the on-disk
code-object cache (_kcache/) ahead of time.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libcgtp.so")
BUILD = os.path.join(HERE, "_build")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          # packed FP32 instructions stay off for all device code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-Wno-format-security"]


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    subprocess.check_call(cmd)
    return obj


def build(verbose: bool = True, out: str = OUT, build_dir: str = BUILD, extra=()) -> str:
    """Compile every source and link the shared library at `out`; `extra`
    flags go to every compile and the link (e.g. host-only sanitizers for a
    test build: each -fsanitize= after -Xarch_host)."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".cpp", ".hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, extra), srcs))
    tmp = out + f".tmp{os.getpid()}"
    subprocess.check_call([HIPCC, *COMMON, *extra, "-shared", *objs, "-o", tmp, "-ldl"])
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def aot_standard_plans(verbose: bool = True) -> None:
    """Fill the code-object cache for the standard workloads (no GPU)."""
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from clebsch_gordan_tensor_cg_amd import binding, workloads\n"
        "binding.precompile_standard_plans()\n" % os.path.dirname(HERE)
    )
    subprocess.check_call([sys.executable, "-c", code])
    if verbose:
        print("code-object cache filled")


if __name__ == "__main__":
    build()
    if "--aot" in sys.argv:
        aot_standard_plans()
