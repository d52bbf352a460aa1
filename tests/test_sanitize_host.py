"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Two programs, each built here with both sanitizers and run to completion:

* ``tests/native/oracle_sanitize.c`` compiles the fp64 oracle into itself and
  runs every oracle entry point on small inputs: every dtype, edge sizes
  (V = 1, N = 0, N = 64, empty batches, a 71-node tree), data errors (NaN,
  all -inf rows, tokens and parents out of range).  Leak checking is on.
* ``tests/native/abi_sanitize.cpp`` links the library with its host code
  instrumented (device code is built as usual) and calls every entry point
  with bad, empty and extreme arguments, each of which must be refused, with
  the documented status, before any HIP call.

A sanitizer report ends the program with a non-zero status and fails the
test.  A third build plants an out-of-bounds read in the oracle driver to
show that the sanitizers are live.
"""
import hashlib
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
BUILD = os.path.join(NATIVE, "_build")
CSRC = os.path.join(ROOT, "rejection_sampling_verify_14_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0", "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
           "OMP_NUM_THREADS": "2"}

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed")


def _digest(paths):
    h = hashlib.sha256()
    for p in sorted(paths):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


def _env(**extra):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(extra)
    return env


def _oracle_exe(tag, *defines):
    os.makedirs(BUILD, exist_ok=True)
    src = os.path.join(NATIVE, "oracle_sanitize.c")
    exe = os.path.join(BUILD, f"oracle_sanitize_{tag}")
    rc, out = _run(["gcc", "-g", "-O1", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", *defines, src, "-o", exe, "-lm"])
    assert rc == 0, out
    return exe


def test_oracle_under_sanitizers():
    rc, out = _run([_oracle_exe("plain")], env=_env())
    assert rc == 0, out
    assert "cases clean" in out


def test_sanitizers_are_live():
    rc, out = _run([_oracle_exe("selftest", "-DSANITIZE_SELFTEST")], env=_env())
    assert rc != 0
    assert "runtime error" in out or "AddressSanitizer" in out, out


def _sanitized_library():
    """libspecverify with its host code instrumented, rebuilt when a source changes."""
    srcs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".h"))]
    srcs.append(os.path.join(ROOT, "include", "specverify.h"))
    key = _digest(srcs)
    out_dir = os.path.join(BUILD, "lib_" + key)
    lib = os.path.join(out_dir, "libsv_san.so")
    if os.path.exists(lib):
        return lib
    if os.path.isdir(BUILD):
        for d in os.listdir(BUILD):
            if d.startswith("lib_"):
                shutil.rmtree(os.path.join(BUILD, d), ignore_errors=True)
    os.makedirs(out_dir, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs, objs = [], []
    for s in ("specverify", "sv_kv", "sv_tree", "sv_draft"):
        obj = os.path.join(out_dir, s + ".o")
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *flags, *san, "-c", os.path.join(CSRC, s + ".hip"), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out = p.communicate()[0]
        assert p.returncode == 0, out
    rc, out = _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *san, *objs, "-o", lib + ".tmp"])
    assert rc == 0, out
    os.replace(lib + ".tmp", lib)
    for o in objs:
        os.remove(o)
    return lib


@pytest.mark.skipif(not os.path.exists(HIPCC) or not os.path.exists(CLANGXX), reason="ROCm compilers needed")
@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="host-only check: run where no GPU is attached")
def test_abi_host_validation_under_sanitizers():
    lib = _sanitized_library()
    d = os.path.dirname(lib)
    exe = os.path.join(d, "abi_sanitize")
    rc, out = _run([CLANGXX, "-g", "-O1", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                    os.path.join(NATIVE, "abi_sanitize.cpp"), "-L", d, "-lsv_san", f"-Wl,-rpath,{d}", "-o", exe])
    assert rc == 0, out
    # the HIP runtime keeps allocations until exit: leaks are checked in the oracle run only
    rc, out = _run([exe], env=_env(ASAN_OPTIONS="detect_leaks=0"))
    assert rc == 0, out
    assert "calls clean" in out
