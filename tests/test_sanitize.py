"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer builds (CPU, no GPU needed).

* The library's C ABI (draft_head_verification_amd/csrc/api.hip) with host sanitizers, linked
  against CPU stand-ins for its kernel launchers (tests/sanitize/launch_stubs.hip), driven by
  tests/sanitize/host_checks.cpp: argument rejection, size queries at the limits, the carving of
  every workspace region (the stand-ins write each region in full into buffers of exactly the
  queried size) and the launch sequence of every call.
* The oracle (oracle/dspark_oracle.c) built with the same sanitizers and driven by
  tests/sanitize/oracle_checks.c over every entry point, both dtypes and samplers, greedy,
  sampled, ragged and empty drafts, the recurrent head and its argument checks.
A sanitizer report makes the program exit nonzero (no recovery).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "draft_head_verification_amd", "csrc")
INC = os.path.join(ROOT, "include")
HIPCC = "/opt/rocm/bin/hipcc"
# host-side sanitizers only: each flag goes to the host compilation of a HIP source
HOST_SAN = []
for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer"):
    HOST_SAN += ["-Xarch_host", flag]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    out = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in ln)
    return res.returncode, out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_api_under_sanitizers(tmp_path):
    common = [HIPCC, "-O1", "-g", "-std=c++17", "-I", INC, "-I", CSRC, *HOST_SAN]
    objs = []
    for name, src, extra in (("api", os.path.join(CSRC, "api.hip"), ["--offload-arch=gfx950"]),
                             ("stubs", os.path.join(SAN, "launch_stubs.hip"),
                              ["--offload-arch=gfx950"]),
                             ("driver", os.path.join(SAN, "host_checks.cpp"), [])):
        obj = str(tmp_path / f"{name}.o")
        rc, out = _run([*common, *extra, "-c", src, "-o", obj])
        assert rc == 0, out
        objs.append(obj)
    exe = str(tmp_path / "host_checks")
    rc, out = _run([HIPCC, "--offload-arch=gfx950", *HOST_SAN, *objs, "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV, timeout=300)
    assert rc == 0 and "host checks: 0 failures" in out, out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    rc, out = _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    os.path.join(SAN, "oracle_checks.c"), os.path.join(ROOT, "oracle", "dspark_oracle.c"),
                    "-o", exe, "-lm"])
    assert rc == 0, out
    env = dict(ENV, ASAN_OPTIONS="detect_leaks=1")
    rc, out = _run([exe], env=env, timeout=300)
    assert rc == 0 and "oracle checks: 0 failures" in out, out
