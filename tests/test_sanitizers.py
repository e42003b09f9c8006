"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the host code, run on the CPU.

* the C oracle with tests/sanitize/oracle_checks.c: every oracle function on small inputs in
  buffers of exactly the documented sizes (gcc, no OpenMP);
* the library's host code (the C-ABI checks, the workspace-size arithmetic, the launchers) with
  tests/sanitize/abi_checks.cpp: calls that each fail a host-side check before any HIP call,
  and the workspace-size functions over large shapes.  The device code is built as usual;
  the sanitizers instrument the host side only (each one given to the host compiler alone).

Any invalid access or undefined operation aborts the driver, which fails the test.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_sparse_08_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# host-side sanitizers for hipcc: -Xarch_host right before each one
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all".split()
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r.stdout


@pytest.mark.timeout(300)
def test_oracle_under_sanitizers():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_checks")
        _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-Wno-unknown-pragmas", os.path.join(HERE, "oracle_checks.c"), os.path.join(ROOT, "oracle", "csa_oracle.c"),
              "-lm", "-o", exe], d)
        out = _run([exe], d)
        assert "0 failures" in out, out


@pytest.mark.timeout(600)
def test_c_abi_host_code_under_sanitizers():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *HOST_SAN, "-fno-gpu-sanitize",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
             f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    srcs = [os.path.join(CSRC, f) for f in ("api.cpp", "compress.hip", "indexer.hip", "topk.hip", "mqa.hip", "rope.hip")]
    srcs.append(os.path.join(HERE, "abi_checks.cpp"))
    with tempfile.TemporaryDirectory() as d:
        procs, objs = [], []
        for s in srcs:
            o = os.path.join(d, os.path.splitext(os.path.basename(s))[0] + ".o")
            objs.append(o)
            procs.append(subprocess.Popen([HIPCC, *flags, "-x", "hip", "-c", s, "-o", o], cwd=d,
                                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
        for p, s in zip(procs, srcs):
            _, err = p.communicate()
            assert p.returncode == 0, f"{s}: {err[-4000:]}"
        exe = os.path.join(d, "abi_checks")
        _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
              "-fsanitize=undefined", *objs, "-o", exe], d)
        out = _run([exe], d)
        assert " 0 failures" in out, out
