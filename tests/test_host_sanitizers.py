"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two host-only builds, made here with gcc/g++:
  - the oracle (oracle/oracle.c) with -fsanitize=address,undefined;
  - the C ABI's argument validation (fa_capi.cpp and the shared size header)
    with the same flags, linked against tests/host_dispatch_stub.cpp in place
    of the kernels (the validation tests make invalid calls only, so nothing
    reaches a dispatch function).
The oracle's pin suites and the C ABI's host tests then run in a subprocess
with the sanitizer runtimes preloaded (python itself is not instrumented);
any report aborts that process.  A copy of the oracle with one planted
out-of-bounds write must be caught, which shows the build is instrumented.
Device code is not covered: sanitizers are not available for it here.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_12_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined", "-g"]
ORACLE_SUITES = ["tests/test_oracle_pins.py", "tests/test_oracle_tiling.py", "tests/test_oracle_decode.py",
                 "tests/test_oracle_ext.py", "tests/test_oracle_blocks.py", "tests/test_oracle_prefill.py",
                 "tests/test_oracle_fp8.py", "tests/test_oracle_bwd.py"]


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def san_env(tmp_path_factory):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc's sanitizer runtimes are not installed")
    d = tmp_path_factory.mktemp("san")
    capi = str(d / "libfa_capi_san.so")
    cmd = ["g++", "-O1", "-std=c++17", "-fPIC", "-shared"] + SAN + [
        "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
        os.path.join(CSRC, "fa_capi.cpp"), os.path.join(ROOT, "tests", "host_dispatch_stub.cpp"),
        "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", capi]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ)
    env.update(LD_PRELOAD="%s:%s" % (asan, ubsan), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", ORACLE_EXTRA_CFLAGS=" ".join(SAN),
               FA_HOST_CAPI_LIB=capi, PYTHONDONTWRITEBYTECODE="1")
    return d, env


def _pytest(env, files, extra_env=None):
    e = dict(env)
    e.update(extra_env or {})
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"]
                          + files, cwd=ROOT, env=e, capture_output=True, text=True, timeout=900)


def test_oracle_pins_under_sanitizers(san_env):
    d, env = san_env
    src = d / "oracle.c"
    src.write_text(open(os.path.join(ROOT, "oracle", "oracle.c")).read())
    res = _pytest(env, ORACLE_SUITES, {"ORACLE_TEST_SOURCE": str(src)})
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert os.path.exists(str(src)[:-2] + ".so"), "the sanitized oracle was not built"


def test_capi_validation_under_sanitizers(san_env):
    d, env = san_env
    res = _pytest(env, ["tests/test_capi_host.py"])
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]


def test_planted_overflow_is_caught(san_env):
    d, env = san_env
    text = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    anchor = "int oracle_widen("
    assert anchor in text
    body = text.index("{", text.index(anchor))
    # one write past the end of the output array on every call
    planted = text[:body + 1] + "\n    if (dst && n > 0) dst[n] = 0.0;\n" + text[body + 1:]
    src = d / "oracle_planted.c"
    src.write_text(planted)
    # -s: the sanitizer's report goes to the process's own stderr
    res = _pytest(env, ["-s", "tests/test_oracle_pins.py", "-k", "widen"], {"ORACLE_TEST_SOURCE": str(src)})
    assert res.returncode != 0, "the planted out-of-bounds write went unnoticed"
    assert "AddressSanitizer" in res.stdout + res.stderr
