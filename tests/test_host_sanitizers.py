"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU).

Every source of libgq.so is compiled host-only with both sanitizers and linked
against a stand-in for the HIP runtime (tests/asan/hip_stub.c for the load-time
registration calls, plus generated traps for every other runtime entry point
the objects reference: each aborts with its name).  tests/asan/abi_validation.c
then drives the C ABI through the invalid-argument cases of the ctypes tests
and through sweeps of extreme sizes with NULL pointers.  A sanitizer report, a
wrong code or a call that reaches the runtime fails the run.

Two controls keep this honest: a tiny program with a signed overflow and one
with a heap overrun must be caught by the same flags, and a call that passes
validation must end in a runtime trap.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

from gguf_quant_matmul_amd.build import CSRC, SOURCES

HERE = os.path.dirname(os.path.abspath(__file__))
ASAN_DIR = os.path.join(HERE, "asan")
INCLUDE = os.path.join(HERE, "..", "include")
LLVM = "/opt/rocm/llvm/bin"
CLANG, CLANGXX = os.path.join(LLVM, "clang"), os.path.join(LLVM, "clang++")
# host-only flags: no device code is compiled, so nothing here reaches a GPU
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
HOST_SAN = [f for s in SAN for f in ("-Xarch_host", s)]
RUN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
REGISTERED = {"__hipRegisterFatBinary", "__hipUnregisterFatBinary", "__hipRegisterFunction",
              "__hipRegisterVar"}

pytestmark = pytest.mark.skipif(
    not (os.access(CLANGXX, os.X_OK) and shutil.which("nm")
         and glob.glob("/opt/rocm/llvm/lib/clang/*/lib/*/libclang_rt.asan*")),
    reason="ROCm clang with the sanitizer runtimes is not installed")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def _compile_host_only(src, out_dir):
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    _run([CLANGXX, "-x", "hip", "--offload-host-only", "--offload-arch=gfx950", "-O1", "-g",
          "-std=c++17", "-fPIC", "-w", *HOST_SAN, "-c", os.path.join(CSRC, src), "-o", obj])
    return obj


def _runtime_stand_in(objs, out_dir):
    """Definitions for every HIP symbol the objects leave undefined: an empty
    code-object image per translation unit and a trap per runtime call."""
    nm = _run(["nm", "-u", *objs]).stdout
    undefined = {p[1] for p in (line.split() for line in nm.splitlines())
                 if len(p) == 2 and p[0] == "U"}
    lines = ["#include <stdio.h>", "#include <stdlib.h>"]
    for s in sorted(undefined):
        if s.startswith("__hip_fatbin_"):
            lines.append(f"const unsigned char {s}[16] __attribute__((aligned(16))) = {{0}};")
        elif s.startswith(("hip", "__hip")) and s not in REGISTERED:
            lines.append(f'void {s}(void) {{ fputs("HIP runtime call {s} reached\\n", stderr); '
                         "abort(); }")
    path = os.path.join(out_dir, "hip_traps.c")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("host_sanitizers"))
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda s: _compile_host_only(s, out), SOURCES))
    traps = _runtime_stand_in(objs, out)
    stubs = []
    for c in (os.path.join(ASAN_DIR, "hip_stub.c"), traps):
        o = os.path.join(out, os.path.basename(c)[:-2] + ".o")
        _run([CLANG, "-O1", "-fPIC", "-w", *SAN, "-c", c, "-o", o])
        stubs.append(o)
    lib = os.path.join(out, "libgq_san.so")
    _run([CLANGXX, "-shared", "-fPIC", *objs, *stubs, "-o", lib])
    exe = os.path.join(out, "abi_validation")
    _run([CLANG, "-O1", "-g", *SAN, "-I", INCLUDE, os.path.join(ASAN_DIR, "abi_validation.c"),
          lib, f"-Wl,-rpath,{out}", "-lm", "-o", exe])
    needed = _run(["readelf", "-d", lib]).stdout
    assert "libamdhip64" not in needed, "the sanitizer build must not load the real HIP runtime"
    return exe


def test_abi_validation_under_sanitizers(driver):
    r = subprocess.run([driver], capture_output=True, text=True, env=RUN_ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr


def test_call_past_validation_hits_runtime_trap(driver):
    r = subprocess.run([driver, "--reach-runtime"], capture_output=True, text=True, env=RUN_ENV,
                       timeout=60)
    assert r.returncode != 0 and "HIP runtime call" in r.stderr, r.stdout + r.stderr


@pytest.mark.parametrize("body,report", [
    ("int f(int a) { return a + 1; }\n"
     "int main(int c, char** v) { (void)v; return f(2147483647 - 1 + c) == 0; }",
     "runtime error"),
    ("#include <stdlib.h>\n"
     "int main(int c, char** v) { (void)v; int* p = malloc(4 * sizeof(int));"
     " int r = p[3 + c]; free(p); return r; }",
     "heap-buffer-overflow"),
])
def test_sanitizer_flags_catch_planted_errors(tmp_path, body, report):
    src = tmp_path / "planted.c"
    src.write_text(body)
    exe = str(tmp_path / "planted")
    _run([CLANG, "-O0", "-g", *SAN, str(src), "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, env=RUN_ENV, timeout=60)
    assert r.returncode != 0 and report in r.stderr, r.stderr
