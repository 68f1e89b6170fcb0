"""CPU sanitizer builds (AddressSanitizer + UndefinedBehaviorSanitizer).

- The oracle (oracle/oracle.c) built with gcc's sanitizers, and its pin tests
  (test_oracle_pins, test_oracle_multi, test_oracle_quant) run against it in
  a subprocess with the ASan runtime preloaded.
- The C ABI's host code (the argument checks of api.hip and validate.hip)
  built with the host compiler's sanitizers (device code unchanged), linked
  with the other objects of the library, and test_abi run against it.
Each build is first shown to report a planted out-of-bounds read, so a
silent sanitizer cannot pass for a clean run."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "query_aware_sparse_paged_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]
# host-side sanitizers only: each -fsanitize= applies to the host pass
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0", "UBSAN_OPTIONS": "halt_on_error=1"}

PLANTED = r"""
#include <stdlib.h>
#ifdef __cplusplus
extern "C"
#endif
int planted(int i) { int *a = (int *)malloc(4 * sizeof(int)); int v = a[i]; free(a); return v; }
"""


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, **kw)


def _gcc_asan_runtime():
    p = _run(["gcc", "-print-file-name=libasan.so"]).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _clang_asan_runtime():
    r = _run([HIPCC, "--offload-arch=gfx950", "-print-file-name=libclang_rt.asan-x86_64.so"])
    p = r.stdout.strip()
    if os.path.isabs(p) and os.path.exists(p):
        return p
    for cand in ("/opt/rocm/lib/llvm/lib/clang", "/opt/rocm/llvm/lib/clang"):
        if os.path.isdir(cand):
            for v in sorted(os.listdir(cand)):
                f = os.path.join(cand, v, "lib", "linux", "libclang_rt.asan-x86_64.so")
                if os.path.exists(f):
                    return f
    return None


def _planted_fails(lib, preload):
    """Calls planted(4) (one past a 4-int allocation) through ctypes in a
    subprocess under the sanitizer runtime; True when the run is reported."""
    code = "import ctypes; ctypes.CDLL(%r).planted(4)" % lib
    r = _run([sys.executable, "-c", code], env=dict(os.environ, LD_PRELOAD=preload, **SAN_ENV))
    return r.returncode != 0 and ("AddressSanitizer" in r.stderr or "runtime error" in r.stderr)


def _pytest(files, env):
    r = _run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] + files, cwd=ROOT,
             env=dict(os.environ, **env, **SAN_ENV))
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_and_ubsan(tmp_path):
    rt = _gcc_asan_runtime()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    planted_c = tmp_path / "planted.c"
    planted_c.write_text(PLANTED)
    planted_so = str(tmp_path / "libplanted.so")
    subprocess.check_call(["gcc", "-shared", "-fPIC"] + GCC_SAN + [str(planted_c), "-o", planted_so])
    assert _planted_fails(planted_so, rt), "the sanitizer build did not report a planted out-of-bounds read"
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-Wall",
                           "-shared", "-fPIC"] + GCC_SAN +
                          [os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib, "-lm"])
    _pytest(["tests/test_oracle_pins.py", "tests/test_oracle_multi.py", "tests/test_oracle_quant.py"],
            {"LD_PRELOAD": rt, "QASP_ORACLE_LIB": lib})


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_c_abi_host_checks_under_asan_and_ubsan(tmp_path):
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    planted_cc = tmp_path / "planted.hip"
    planted_cc.write_text(PLANTED)
    planted_so = str(tmp_path / "libplanted.so")
    subprocess.check_call([HIPCC] + HIP_FLAGS + HOST_SAN + ["-shared", str(planted_cc), "-o", planted_so])
    assert _planted_fails(planted_so, rt), "the sanitizer build did not report a planted out-of-bounds read"
    from query_aware_sparse_paged_amd import build as qbuild
    from concurrent.futures import ThreadPoolExecutor

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        san = HOST_SAN if src in ("api.hip", "validate.hip") else []
        r = _run([HIPCC] + HIP_FLAGS + san + ["-c", os.path.join(CSRC, src), "-o", obj])
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with ThreadPoolExecutor(max(1, min(len(qbuild.SOURCES), os.cpu_count() or 1))) as ex:
        objs = list(ex.map(compile_one, qbuild.SOURCES))
    vs = tmp_path / "exports.map"
    vs.write_text("{ global: qasp_*; local: *; };\n")
    lib = str(tmp_path / "libqasp_san.so")
    r = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,--version-script=" + str(vs)] + HOST_SAN +
             ["-o", lib] + objs)
    assert r.returncode == 0, r.stderr[-2000:]
    _pytest(["tests/test_abi.py"], {"LD_PRELOAD": rt, "QASP_LIB": lib})
