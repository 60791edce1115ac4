"""AddressSanitizer / UndefinedBehaviorSanitizer runs on the CPU.

- The oracle (oracle/dsa_oracle.c) built with gcc under both sanitizers and
  driven by tests/native/oracle_sanitize.c through every entry point.
- libdsa's host code (argument validation, workspace plans, size queries)
  built with the sanitizers on the host side only (the device code is compiled
  as usual and never runs) and driven by tests/native/host_sanitize.cpp with
  arguments the validation rejects before any HIP call.
A sanitizer report aborts the program, which fails the test."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, **kw)
    text = r.stdout.decode(errors="replace")
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{text[-4000:]}"
    return text


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", *SAN, "-Wall", "-Wno-unknown-pragmas",
          os.path.join(NATIVE, "oracle_sanitize.c"), os.path.join(ROOT, "oracle", "dsa_oracle.c"), "-lm", "-o", exe])
    out = _run([exe], env=ENV)
    assert "oracle sanitizer run ok" in out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_library_host_code_under_sanitizers(tmp_path):
    host_san = [f for s in SAN for f in ("-Xarch_host", s)]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "sparse_attention_14_amd", "csrc")]
    common = ["-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", *host_san, *inc]
    srcs = sorted(f for f in os.listdir(os.path.join(ROOT, "sparse_attention_14_amd", "csrc")) if f.endswith(".hip"))
    objs = [str(tmp_path / (s + ".o")) for s in srcs]

    def compile_one(i):
        src = os.path.join(ROOT, "sparse_attention_14_amd", "csrc", srcs[i])
        return _run([HIPCC, "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                     *common, "-c", src, "-o", objs[i]])

    with ThreadPoolExecutor(max_workers=4) as ex:
        list(ex.map(compile_one, range(len(srcs))))
    drv = str(tmp_path / "drv.o")
    _run([HIPCC, *common, "-x", "c++", "-c", os.path.join(NATIVE, "host_sanitize.cpp"), "-o", drv])
    exe = str(tmp_path / "host_san")
    _run([HIPCC, "--offload-arch=gfx950", *host_san, *objs, drv, "-o", exe])
    out = _run([exe], env=ENV)
    assert "host sanitizer run ok" in out
