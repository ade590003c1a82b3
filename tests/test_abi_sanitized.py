"""The host code of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer: the library
is rebuilt with the host side of every source instrumented (device code unchanged) and the
host-side ABI tests (tests/test_abi_host.py: every argument error, the workspace sizes and
plans) run against it in a child process with the sanitizer runtime loaded first.  Any
report fails the run.  CPU only: no call reaches a kernel launch."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_host_under_sanitizers(tmp_path):
    from attention_sink_softmax_amd import build as b

    hipcc = b.HIPCC
    rt = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    if not os.path.exists(rt):
        pytest.skip("no ASan runtime next to hipcc")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
           "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan"]
    objs = []
    for src in b.SOURCES:
        o = str(tmp_path / src.replace(".hip", ".o"))
        b._run([hipcc, *b.FLAGS, *b.EXTRA.get(src, []), *san, "-c", os.path.join(b.CSRC, src), "-o", o])
        objs.append(o)
    lib = str(tmp_path / "libsinkattn_san.so")
    b._run([hipcc, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", *san, *objs, "-o", lib])
    env = dict(os.environ, LD_PRELOAD=rt, SINKATTN_TEST_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
