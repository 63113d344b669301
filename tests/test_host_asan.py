"""Host AddressSanitizer runs (CPU only):
  - the library's host code (argument checks, the packer, the expert-cache policy)
    built with the sanitizer on its host side only (the GPU code objects are built
    as usual), under the CPU tests that call it: test_lib_host.py, test_cache_policy.py;
  - the fp64 oracle built with the sanitizer, under its pins: test_oracle_pins.py.
Each runs in a child process with the matching ASan runtime preloaded (clang's for
the hipcc build, gcc's for the oracle); any ASan report or test failure fails here."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "quantized_mixture_experts_bit_amd")

pytestmark = pytest.mark.timeout(900)


def _runtime(compiler, name):
    p = subprocess.run([compiler, "-print-file-name=" + name], stdout=subprocess.PIPE, text=True).stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip("%s has no %s here" % (compiler, name))
    return p


def _child(tests, env_extra, preload):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] + tests
    res = subprocess.run(cmd, cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                         timeout=800)
    out = res.stdout
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]


def test_library_host_code_under_asan(tmp_path):
    sys.path.insert(0, PKG)
    from quantized_mixture_experts_bit_amd import build as qbuild
    lib = str(tmp_path / "libqmoe_asan.so")
    # the sanitizer applies to the host side of every source only
    cmd = (["hipcc"] + [f for f in qbuild.FLAGS] +
           ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-o", lib] + qbuild.SOURCES)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout[-3000:]
    preload = _runtime("/opt/rocm/llvm/bin/clang", "libclang_rt.asan-x86_64.so")
    _child(["tests/test_lib_host.py", "tests/test_cache_policy.py"], {"QMOE_LIB": lib}, preload)


def test_oracle_under_asan(tmp_path):
    sys.path.insert(0, ROOT)
    import oracle
    lib = oracle.build(out=str(tmp_path / "liboracle_asan.so"),
                       extra_flags=["-fsanitize=address", "-fno-omit-frame-pointer"])
    preload = _runtime("gcc", "libasan.so")
    _child(["tests/test_oracle_pins.py"], {"QMOE_ORACLE_LIB": lib}, preload)
