"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle (gcc) is rebuilt with -fsanitize=address,undefined into a temporary
directory and the oracle's own pin tests run against it in a child process with
the sanitizer runtimes preloaded; any report aborts the child.  The HIP
library's host code (argument checks, workspace sizing, status strings) is
checked the same way when its sanitizer build exists
(``python -m gemm_block_quant_amd.build --sanitize``, which takes minutes and is
therefore not done here).
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_LIB = os.path.join(ROOT, "gemm_block_quant_amd", "_asan", "libquantgemm.so")


def _gcc_runtime(name):
    out = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def _run_pytest(env_extra, tests, tmp_path):
    log = str(tmp_path / "sanlog")
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:log_path=" + log
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:log_path=" + log
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + tests
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = sorted(glob.glob(log + "*"))
    text = "".join(open(p).read() for p in reports)
    assert not reports, "sanitizer report:\n" + text[:4000]
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]


def test_oracle_under_asan_ubsan(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    import oracle
    lib = oracle.build(out=str(tmp_path / "liboracle_san.so"), sanitize=True)
    _run_pytest({"LD_PRELOAD": asan + " " + ubsan, "QG_ORACLE_LIB": lib},
                ["tests/test_oracle.py", "tests/test_specials_host.py"], tmp_path)


def test_library_host_code_under_asan_ubsan(tmp_path):
    if not os.path.exists(SAN_LIB):
        pytest.skip("sanitizer build of the library not present (python -m gemm_block_quant_amd.build --sanitize)")
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang AddressSanitizer runtime not found")
    _run_pytest({"LD_PRELOAD": rt[-1], "QUANTGEMM_LIB": SAN_LIB}, ["tests/test_abi.py"], tmp_path)
