"""Host-side argument validation of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer.

Every library source is compiled with both sanitizers on its host code only
(the device code is built as usual and never runs), linked with
tests/sanitize/abi_checks.cpp, and run as a child process.  The checks pass only invalid arguments, which every entry
point must reject on the host before any HIP call, so no GPU is needed."""
import hashlib
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from post_weight_quantization_layer_amd import build as LB

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _build():
    srcs = [os.path.join(LB.CSRC, s) for s in LB.SOURCES]
    heads = [os.path.join(LB.CSRC, "common.h"), os.path.join(LB.INCLUDE, "gptq.h")]
    tag = _digest(srcs + heads + [DRIVER])
    exe = os.path.join(OUT, f"abi_checks_{tag}")
    if os.path.exists(exe):
        return exe
    os.makedirs(OUT, exist_ok=True)
    cc = LB.hipcc()
    common = [f"--offload-arch={LB.ARCH}", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              f"-I{LB.INCLUDE}", f"-I{LB.CSRC}", *SAN]

    def one(src):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        r = subprocess.run([cc, *common, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr
        return obj

    with ThreadPoolExecutor(8) as ex:
        objs = list(ex.map(one, srcs + [DRIVER]))
    r = subprocess.run([cc, f"--offload-arch={LB.ARCH}", *SAN, "-o", exe, *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
def test_abi_validation_under_asan_and_ubsan():
    exe = _build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ok: 0 failure(s)" in out
    assert "runtime error" not in out and "AddressSanitizer" not in out
