"""Build the HIP library ``libkvc.so`` in-tree for gfx950.

Usage: ``python -m kv_cached_gqa_append_amd.build`` (or ``build()``).  Always
recompiles.  The library lands next to this file, where the binding loads it.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvc.so")
SOURCES = ["kernels.hip", "kvc_api.cpp", "layout.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wextra",
    "-Werror",
    # packed FP32 instructions stay off (gfx950 code generation choice)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


_NOISE = "is not a recognized feature for this target"


def _stderr(res):
    return "\n".join(l for l in (res.stderr or "").splitlines() if _NOISE not in l)


def build(verbose: bool = False) -> str:
    """Compile libkvc.so and check the device assembly of the kernels.

    The assembly check (``asm_check``) runs on a device-only compile of
    kernels.hip made with the same flags, in parallel with the library build;
    a problem in it fails the build and leaves any older library in place.
    """
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    asm = os.path.join(HERE, "_kernels.s")
    cmd = [HIPCC] + FLAGS + ["-o", tmp] + srcs
    dev_flags = [f for f in FLAGS if f not in ("-shared", "-fPIC")]
    cmd_s = [HIPCC] + dev_flags + ["-Wno-unused-command-line-argument", "--cuda-device-only", "-S", "-o", asm,
                                   os.path.join(CSRC, "kernels.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    p_lib = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    res_s = subprocess.run(cmd_s, capture_output=True, text=True)
    out, errs = p_lib.communicate()
    res = subprocess.CompletedProcess(cmd, p_lib.returncode, out, errs)
    err = _stderr(res)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if res_s.returncode != 0:
        raise RuntimeError(f"hipcc -S failed ({res_s.returncode}):\n{_stderr(res_s)}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    from . import asm_check
    with open(asm) as f:
        n, problems = asm_check.check_assembly(f.read())
    os.remove(asm)
    if n == 0 or problems:
        os.remove(tmp)
        raise RuntimeError("device assembly check failed:\n" + "\n".join(
            problems or ["no kernel with tile loads found"]))
    if verbose:
        print(f"assembly check: {n} kernels with hand-placed waits, no problems", flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
