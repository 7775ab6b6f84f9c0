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
# Debug build: every kernel fills its LDS with NaN bytes before first use
# (FA_DEBUG_POISON), so a read of LDS the launch never wrote shows up as NaN
# in the outputs, and every entry point waits for its stream before it
# returns (FA_DEBUG_SYNC), so a device fault is reported by the call that
# caused it.  Tests only; the product loads LIB.
LIB_POISON = os.path.join(HERE, "libfa_poison.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("fa_fwd.hip", "fa_bwd.hip", "fa_fp8.hip",
                                                    "fa_decode.hip", "fa_capi.cpp")]

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


def _compile(hipcc, src, obj, extra=()):
    """One translation unit to a position-independent object; returns (src, rc, messages)."""
    flags = [f for f in HIPCC_FLAGS if f != "-shared"] + list(extra)
    res = subprocess.run([hipcc] + flags + ["-c", src, "-o", obj], capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    return src, res.returncode, msgs


def build(verbose: bool = False, poison: bool = False) -> str:
    """Compile libfa.so (always recompiles; one process per source file) and return its path.

    poison=True builds the debug library libfa_poison.so instead (LDS poisoning, and a
    stream synchronisation at the end of every call)."""
    extra = ["-DFA_DEBUG_POISON", "-DFA_DEBUG_SYNC"] if poison else []
    target = LIB_POISON if poison else LIB
    import concurrent.futures
    import shutil
    import tempfile
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmpdir = tempfile.mkdtemp(prefix="fa_build_")
    try:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in SOURCES]
        if verbose:
            print(" ".join([hipcc] + HIPCC_FLAGS + extra + ["-c"] + SOURCES), flush=True)
        workers = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(lambda so: _compile(hipcc, *so, extra=extra), zip(SOURCES, objs)))
        for src, rc, msgs in results:
            if rc != 0:
                raise RuntimeError("hipcc failed on %s (%d):\n%s" % (src, rc, "\n".join(msgs)))
            if verbose and msgs:
                print("\n".join(msgs), flush=True)
        tmp = target + ".tmp%d" % os.getpid()
        res = subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp],
                             capture_output=True, text=True)
        if res.returncode != 0:
            if os.path.exists(tmp):
                os.remove(tmp)
            raise RuntimeError("link failed (%d):\n%s" % (res.returncode, res.stdout + res.stderr))
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    # the library must load with every symbol resolved (a kernel whose host
    # launch stub was not emitted shows up here, not at the first call)
    chk = subprocess.run([sys.executable, "-c", "import ctypes, sys; ctypes.CDLL(sys.argv[1])", tmp],
                         capture_output=True, text=True)
    if chk.returncode != 0:
        os.remove(tmp)
        raise RuntimeError("built library does not load:\n" + chk.stderr)
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build(verbose="-v" in sys.argv, poison=True))
