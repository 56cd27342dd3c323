"""The oracle's C (manual allocation and pointer arithmetic) and the C ABI's
host code (argument validation, workspace layout) run once under
AddressSanitizer and UndefinedBehaviorSanitizer on the CPU: the oracle pins
and the coarse-check pins against an instrumented oracle, and the ABI tests
against a library whose host code is instrumented.  Any report fails the
run (abort on error)."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_long_context_means_amd")


def _run(args, env, cwd=ROOT):
    full = dict(os.environ)
    full.update(env)
    r = subprocess.run(args, cwd=cwd, env=full, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-4000:] + r.stderr[-4000:]


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    rc, out = _run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-o", lib,
                    os.path.join(ROOT, "oracle", "mpattn_oracle.c"), "-lm"], {})
    assert rc == 0, out
    pre = ":".join(subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True).stdout.strip()
                   for n in ("libasan.so", "libubsan.so"))
    rc, out = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                    "tests/test_oracle_pins.py", "tests/test_coarse_check.py"],
                   {"LD_PRELOAD": pre, "MPATTN_ORACLE_LIB": lib,
                    "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1", "UBSAN_OPTIONS": "halt_on_error=1"})
    assert rc == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out


def test_abi_host_code_under_asan_ubsan(tmp_path):
    objs = sorted(glob.glob(os.path.join(PKG, "_build", "*.o")))
    if not any(o.endswith("unit.o") for o in objs):
        pytest.skip("the library's objects are not built")
    sys.path.insert(0, PKG)
    import _build

    san = str(tmp_path / "api_san.o")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in _build.FLAGS if f != "-O3"] + ["-O1", "-g"]
    rc, out = _run([_build.HIPCC, *flags, *host_san, "-c", os.path.join(PKG, "csrc", "api.hip"), "-o", san], {})
    assert rc == 0, out
    lib = str(tmp_path / "libmpattn_san.so")
    others = [o for o in objs if not o.endswith("api.o")]
    rc, out = _run([_build.HIPCC, f"--offload-arch={_build.ARCH}", "-shared", "-fPIC", "-fsanitize=address,undefined",
                    "-shared-libsan", "-o", lib, san, *others], {})
    assert rc == 0, out
    rt = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt:
        pytest.skip("no clang AddressSanitizer runtime")
    rc, out = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_abi.py"],
                   {"LD_PRELOAD": rt[0], "MPATTN_LIB": lib,
                    "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1", "UBSAN_OPTIONS": "halt_on_error=1"})
    assert rc == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
