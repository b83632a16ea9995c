"""The host layer of libgdn (its argument checks and workspace arithmetic) and the C oracle,
built with AddressSanitizer and UndefinedBehaviorSanitizer (host code only; errors abort) and
driven by the programs in tests/sanitize/: every entry point with arguments its checks
reject, sizes at the edges of int and 64-bit arithmetic included, and the oracle on small
packed problems through all of its branches. No device is used."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "gated_delta_rule_42_amd", "csrc")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", os.path.join(SAN, "oracle_driver.c"),
         os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-lm", "-o", exe], str(tmp_path))
    assert "all checks passed" in run([exe], str(tmp_path))


def test_host_layer_under_sanitizers(tmp_path):
    """gdn_api.hip and gdn_noalloc.hip with host-side sanitizers, linked with the other objects
    of the library as build() compiled them."""
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    from gated_delta_rule_42_amd import build as B

    objdir = os.path.join(ROOT, "gated_delta_rule_42_amd", "build")
    B.build()   # up-to-date objects of the kernels
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [HIPCC, *B.HIPCC_FLAGS, "-g", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for src in ("gdn_api.hip", "gdn_noalloc.hip"):
        o = str(tmp_path / (src + ".o"))
        run([*flags, *san, "-c", os.path.join(CSRC, src), "-o", o], str(tmp_path))
        objs.append(o)
    others = [os.path.join(objdir, os.path.basename(src)[:-4] + ".o") for src in B.sources()
              if os.path.basename(src) not in ("gdn_api.hip", "gdn_noalloc.hip")]
    assert others and all(os.path.exists(o) for o in others), "library objects missing"
    drv = str(tmp_path / "abi_driver.o")
    run([*flags, *san, "-c", os.path.join(SAN, "abi_driver.cpp"), "-o", drv], str(tmp_path))
    exe = str(tmp_path / "abi_driver")
    run([HIPCC, f"--offload-arch={B.ARCH}", *san, drv, *objs, *others, "-o", exe], str(tmp_path))
    assert "all checks passed" in run([exe], str(tmp_path))
