"""Host-side sanitizers: the CPU oracle and the host code of the C ABI (argument
validation, workspace and index layouts), built with AddressSanitizer and
UndefinedBehaviorSanitizer, run the host test modules in a child process.

The HIP library is built with the sanitizers on its host pass only (each
-fsanitize= after -Xarch_host); its device code is unchanged and never runs
here: the child process only calls entry points that fail validation or
compute sizes.  Both libraries use clang's shared sanitizer runtime, which the
child process preloads.  Skipped where a GPU is visible (the host tests then
skip their no-GPU checks) or where the toolchain is missing.
"""
import concurrent.futures
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lsh_sampled_sparse_centered_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-shared-libsan"]


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


pytestmark = pytest.mark.skipif(_gpu_visible() or not (os.path.exists(CLANG) and os.path.exists(HIPCC) and RUNTIME),
                                reason="host sanitizer builds run on the CPU-only host with the ROCm toolchain")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-2000:], r.stderr[-4000:])


def _build(tmp):
    oracle_so = os.path.join(tmp, "libmp_oracle.so")
    _run([CLANG, "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared", *SAN, "-o", oracle_so,
          os.path.join(ROOT, "oracle", "mp_oracle.c"), "-lm"])
    host_san = [a for f in SAN for a in ("-Xarch_host", f)]
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             "-Wno-unused-command-line-argument", *host_san]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(tmp, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        list(ex.map(lambda so: _run([HIPCC, *flags, "-c", so[0], "-o", so[1]]), zip(srcs, objs)))
    lib_so = os.path.join(tmp, "libmagicpig.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *host_san, "-o", lib_so, *objs])
    return oracle_so, lib_so


DRIVER = """
import sys
sys.path.insert(0, {root!r})
import oracle
import lsh_sampled_sparse_centered_amd as mp
oracle._LIB = {oracle_so!r}
mp.LIB_PATH = {lib_so!r}
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu and not slow",
                      {pins!r}, {abi!r}, {planes!r}]))
"""


def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    oracle_so, lib_so = _build(str(tmp_path))
    drv = tmp_path / "drv.py"
    drv.write_text(DRIVER.format(root=ROOT, oracle_so=oracle_so, lib_so=lib_so,
                                 pins=os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                                 abi=os.path.join(ROOT, "tests", "test_abi_host.py"),
                                 planes=os.path.join(ROOT, "tests", "test_planes_host.py")))
    env = dict(os.environ, LD_PRELOAD=RUNTIME[-1], ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, str(drv)], capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-6000:]
    assert "passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]
