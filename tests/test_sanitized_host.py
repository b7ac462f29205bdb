"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The host side of liblmhead.so (argument checks, size and layout arithmetic,
workspace carving, status strings) is built with -fsanitize=address,undefined
and exercised two ways: by the plain C client (tests/c_client/abi_client.c,
itself built with the sanitizers) and by the ABI tests of tests/test_abi.py run
in a child interpreter with the sanitizer runtime loaded first. None of these
calls launches a kernel (the device code is built but never runs, and has no
sanitizer here). Any report, or a test failure, fails the test.
"""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lm_head_log_amd", "csrc")
SRCS = [os.path.join(CSRC, f) for f in ("lmhead.hip", "logits_rows.hip", "mfma_probe.hip")]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")

# each sanitizer flag applies to the host compilation only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
    "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
}


def _asan_runtime():
    hits = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    rt = _asan_runtime()
    if not os.path.exists(HIPCC) or not os.path.exists(CLANG) or rt is None:
        pytest.skip("hipcc, clang or the ASan runtime is missing")
    d = tmp_path_factory.mktemp("sanitized")
    lib = str(d / "liblmhead.so")
    common = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-fvisibility=hidden", *SAN, "-I", os.path.join(ROOT, "include")]
    # one object per source, compiled side by side, then one link
    objs, procs = [], []
    for src in SRCS:
        obj = str(d / (os.path.basename(src) + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen(common + ["-c", src, "-o", obj], stdout=subprocess.PIPE,
                                      stderr=subprocess.PIPE, text=True))
    for p in procs:
        _, err = p.communicate(timeout=900)
        assert p.returncode == 0, err[-4000:]
    r = subprocess.run(common + ["-shared", "-shared-libasan", "-o", lib, *objs],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    # the host code really is instrumented: it calls into both runtimes
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    return {"dir": str(d), "lib": lib, "rt": rt}


def _env(s, extra=None):
    env = dict(os.environ)
    env.update(SAN_ENV)
    # the runtime must come first; whatever was preloaded stays after it
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = s["rt"] + (":" + pre if pre else "")
    env["LD_LIBRARY_PATH"] = os.path.dirname(s["rt"]) + ":" + env.get("LD_LIBRARY_PATH", "")
    env.update(extra or {})
    return env


def test_c_client_under_sanitizers(sanitized):
    exe = os.path.join(sanitized["dir"], "abi_client")
    src = os.path.join(ROOT, "tests", "c_client", "abi_client.c")
    r = subprocess.run([CLANG, "-std=c11", "-Wall", "-Werror", "-g", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", "-shared-libasan",
                        "-I", os.path.join(ROOT, "include"), src, "-o", exe,
                        "-L", sanitized["dir"], "-llmhead", f"-Wl,-rpath,{sanitized['dir']}",
                        f"-Wl,-rpath,{os.path.dirname(sanitized['rt'])}"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ)
    env.update(SAN_ENV)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "all checks passed" in r.stdout
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]


def test_abi_tests_under_sanitizers(sanitized):
    # the binding checks that import torch stay out: torch is not built for
    # the sanitizer runtime; every library call of the ABI tests stays in
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        "-k", "not binding_rejects_cpu_tensors"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT,
                       env=_env(sanitized, {"LMHEAD_LIB": sanitized["lib"]}))
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in r.stdout
