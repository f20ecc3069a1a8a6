"""Address and undefined-behaviour sanitizer runs on the CPU.

Two host-only builds, each run as its own process so that a sanitizer report
aborts it with a non-zero status:
  * the fp64 oracle (``oracle/oracle.c``) driven by ``sanitize/oracle_fuzz.c``
    with exactly sized buffers (out-of-bounds reads or writes, overflow);
  * the C ABI's host side (``capi.hip`` and the plans in ``plan.cpp``, built
    without device code, the kernel launchers replaced by stubs) driven by
    ``sanitize/abi_fuzz.cpp`` with sizes around every documented limit (signed
    overflow in the size products, invalid enum loads, out-of-bounds accesses).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "selective_state_space_70_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=600, **kw)
    out = r.stdout.decode(errors="replace")
    assert r.returncode == 0, "%s\n%s" % (" ".join(cmd), out[-4000:])
    return out


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_fuzz")
    _run([gcc, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-Wall", "-o", exe, os.path.join(HERE, "oracle_fuzz.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    out = _run([exe], env=ENV)
    assert "runtime error" not in out and "ok" in out, out


def test_abi_host_side_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    flags = ["--cuda-host-only", "-O1", "-g", "-std=c++17", "-I" + os.path.join(ROOT, "include"),
             "-I" + CSRC] + san
    srcs = [os.path.join(CSRC, "capi.hip"), os.path.join(CSRC, "plan.cpp"),
            os.path.join(HERE, "launch_stubs.cpp"), os.path.join(HERE, "abi_fuzz.cpp")]
    objs = []
    procs = []
    for src in srcs:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC] + flags + ["-c", src, "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    for p, src in zip(procs, srcs):
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, "%s\n%s" % (src, out.decode(errors="replace")[-4000:])
    exe = str(tmp_path / "abi_fuzz")
    _run([HIPCC] + san + ["-o", exe] + objs)
    out = _run([exe], env=ENV)
    assert "runtime error" not in out and "ok" in out, out
