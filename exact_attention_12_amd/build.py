"""Build step for libfa.so: compiles the gfx950 kernels and the C ABI with hipcc.

Run as ``python -m exact_attention_12_amd.build`` (or through the repository's
``__graft_entry__.build()``).  The library is written next to this file, so it
travels with the source tree.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libfa.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("fa_fwd.hip", "fa_bwd.hip", "fa_fp8.hip", "fa_decode.hip", "fa_capi.cpp")]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU
# instructions; hipcc's host pass warns that it does not know the feature.
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", os.path.join(HERE, "csrc"),
]


def build(verbose: bool = False) -> str:
    """Compile libfa.so (always recompiles) and return its path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, "\n".join(msgs)))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    # the library must load with every symbol resolved (a kernel whose host
    # launch stub was not emitted shows up here, not at the first call)
    chk = subprocess.run([sys.executable, "-c", "import ctypes, sys; ctypes.CDLL(sys.argv[1])", tmp],
                         capture_output=True, text=True)
    if chk.returncode != 0:
        os.remove(tmp)
        raise RuntimeError("built library does not load:\n" + chk.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
