"""Host-code sanitizer runs (CPU only, no GPU needed).

* The oracle (plain C) is rebuilt with AddressSanitizer and
  UndefinedBehaviorSanitizer, and the oracle pins run against that build.
* libflare's host runtime (flare.cpp: argument validation, plans, workspace
  layout, tuning, timing bookkeeping) is rebuilt with the same sanitizers on
  its host code only (the gfx950 kernels are compiled as usual), and the C-ABI
  host checks run against that build.

Each run is a subprocess with the matching ASan runtime preloaded (a Python
interpreter that is not itself instrumented needs the runtime first in its
library list); a sanitizer report fails the run.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def run_py(code: str, preload: str, tmp_path) -> subprocess.CompletedProcess:
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=preload, PYTHONPATH=ROOT)
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=600)


def check(r: subprocess.CompletedProcess):
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]


def test_oracle_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libflare_oracle_san.so")
    src = os.path.join(ROOT, "oracle", "flare_oracle.c")
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
                    "-std=c99", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", src, "-o", lib, "-lm"], check=True)
    preload = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                             check=True).stdout.strip()
    code = (f"import oracle, pytest, sys; oracle._LIB = {lib!r}; oracle.set_threads(2); "
            "sys.exit(pytest.main(['tests/test_oracle_pins.py', '-q', '-x', '-p', 'no:cacheprovider']))")
    check(run_py(code, preload, tmp_path))


def test_host_runtime_under_asan_ubsan(tmp_path):
    from rank_latent_attention_flare_amd import build as B

    B.build()  # the kernel objects the sanitized library links
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    obj = str(tmp_path / "flare_san.o")
    r = subprocess.run([HIPCC, *B.COMMON, *san, "-g", "-x", "hip", "-c", os.path.join(B.CSRC, "flare.cpp"), "-o",
                        obj], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    kernels = [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "flare.cpp"]
    lib = str(tmp_path / "libflare_san.so")
    r = subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={B.ARCH}", *san, "-shared-libasan", obj,
                        *kernels, "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt:
        pytest.skip("clang ASan runtime not found")
    code = (f"import rank_latent_attention_flare_amd.flare as F, pytest, sys; F.LIB_PATH = {lib!r}; "
            "sys.exit(pytest.main(['tests/test_abi_host.py', '-q', '-x', '-p', 'no:cacheprovider']))")
    check(run_py(code, rt[0], tmp_path))
