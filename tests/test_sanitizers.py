"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

Two checking builds, each exercised in a child process with its sanitizer runtime
preloaded (Python itself is not instrumented):
  * the oracle (gcc, -fsanitize=address,undefined) under its pinning tests;
  * the HIP library with the host code instrumented (hipcc -Xarch_host -fsanitize=...)
    under the C-ABI tests, which drive argument validation, workspace sizing and the
    decode-step layout without launching device work.
Any sanitizer report aborts the child, so the test fails on it."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _run(tests, env_extra, tmp_path):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=87"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-p", "no:xdist", "-m", "not gpu"] + tests,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out


def _runtime(compiler, name):
    p = subprocess.run([compiler, f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    if p.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"{name} not found for {compiler}")
    return path


def test_oracle_under_asan_ubsan(tmp_path):
    from oracle import build as ob
    lib = ob.build(sanitize=True, out=str(tmp_path / "liboracle_san.so"))
    asan = _runtime("gcc", "libasan.so")
    _run(["tests/test_oracle_compress.py", "tests/test_oracle_indexer.py",
          "tests/test_oracle_attention.py", "tests/test_oracle_decode.py",
          "tests/test_oracle_bruteforce.py"],
         {"V4A_ORACLE_LIB": lib, "LD_PRELOAD": asan}, tmp_path)


def test_host_abi_under_asan_ubsan(tmp_path):
    from compressed_sparse_attention_v4a_amd import build as hb
    lib = hb.build(sanitize=True, out=str(tmp_path / "libv4a_san.so"),
                   build_dir=str(tmp_path / "obj"))
    clang = os.path.join(os.path.dirname(os.path.realpath(hb.HIPCC)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    asan = _runtime(clang, "libclang_rt.asan-x86_64.so")
    _run(["tests/test_abi.py"], {"V4A_LIB": lib, "LD_PRELOAD": asan}, tmp_path)
