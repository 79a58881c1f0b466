"""The host code under AddressSanitizer, on the CPU.

Two instrumented builds are made in a temporary folder: the oracle
(``dsa_oracle.c``, gcc's sanitizer) and the library with its host code
instrumented (argument validation, workspace sizing and launch set-up;
clang's sanitizer through hipcc).  The oracle pins and the host ABI tests
then run in child processes with the matching sanitizer runtime preloaded;
any report (out-of-bounds access, use after free, double free) fails the
child and so this test.  Leak detection is off: the Python interpreter
itself keeps allocations alive at exit.
"""
import glob
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _gcc_asan_runtime():
    if shutil.which("gcc") is None:
        return None
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _undefined_dynamic(lib):
    out = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    return out.stdout


def _run_pytest(files, env_extra, preload):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join(ROOT, "tests", f) for f in files]]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    return out


@pytest.mark.skipif(_gcc_asan_runtime() is None, reason="gcc's AddressSanitizer runtime is missing")
def test_oracle_pins_under_asan(tmp_path):
    import oracle
    lib = oracle.build_asan(str(tmp_path / "libdsa_oracle_asan.so"))
    assert "__asan_init" in _undefined_dynamic(lib)
    files = sorted(os.path.basename(p) for p in glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    assert files
    out = _run_pytest(files, {"DSA_ORACLE_LIBRARY": lib}, _gcc_asan_runtime())
    assert " passed" in out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and _clang_asan_runtime()),
                    reason="hipcc or clang's AddressSanitizer runtime is missing")
def test_abi_host_under_asan(tmp_path):
    spec = importlib.util.spec_from_file_location(
        "dsa_build_script", os.path.join(ROOT, "sparse_attention_16_amd", "build.py"))
    dsa_build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(dsa_build)
    lib = dsa_build.build_host_asan(str(tmp_path / "asan"))
    assert "__asan_init" in _undefined_dynamic(lib)
    out = _run_pytest(["test_abi_host.py"], {"DSA_LIBRARY": lib}, _clang_asan_runtime())
    assert " passed" in out and "skipped" not in out
