"""The C ABI's host code (argument checks, workspace sizing, error strings)
built with AddressSanitizer and UndefinedBehaviorSanitizer on the host pass
only, linked with the ordinary kernel objects, and driven through the same
host-side calls as test_abi.py in a fresh interpreter under the ASan runtime.
No call reaches a kernel launch (every call fails its checks first or only
queries sizes), so no GPU is needed."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")

CALLS = r"""
import ctypes, sys
sys.path.insert(0, ROOT)
from draft_then_verify_amd import binding as bd
lib = bd.load_library(LIB)
cfg = bd.spec_model_cfg(256, 4, 4, 4, 96, 704, 4096, bd.SPEC_F32, 10000.0, 1e-6)
w = bd.spec_weights()
h = ctypes.c_void_p()
assert lib.spec_model_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)) == -4
assert "head_dim" in bd.spec_last_error()
cfg.head_dim = 64
assert lib.spec_model_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)) == -1
assert lib.spec_model_create(None, None, None) == -1
lib.spec_model_destroy(None)
assert lib.spec_reject_sample(0, 4, 100, 1, None, 1, None, 1, 1, 1, 1, 1, 1 << 20, None) == -1
assert lib.spec_reject_sample(1, 2, 100, 1, None, 1, None, 1, 1, 1, 1, 1, 8, None) == -2
assert lib.spec_softmax_pq(1, 4, 100, float("nan"), 1, 1, 1 << 20, None) == -1
assert lib.spec_sampler_workspace_bytes(5, 0, 151936) > 0 and lib.spec_sampler_workspace_bytes(-1, 0, 8) == 0
kv = bd.spec_kv(1, 1, 1, 2, 16)
assert lib.spec_kv_set_len(ctypes.byref(kv), 3, None, 1, None) == -1
assert lib.spec_verify_forward(None, ctypes.byref(kv), 1, 1, 1, None, 1, 1 << 30, None) == -1
assert lib.spec_workspace_bytes(None, 1, 1, 16) == 0
assert lib.spec_commit_round(0, 4, 1, 1, 1, None, 1, 1, 8, 0, None, None, None, 0, None) == -1
assert lib.spec_ngram_propose(1, 0, 3, 4, 1, None, 8, None, None, 0, None, 1, 1, None, None) == -1
assert lib.spec_linear(7, 0, 1, 1, 1, 1, 1, 1, None, None, None, 0.0, None) == -1
assert lib.spec_linear(1, 0, 16, None, 1, 1, 8, 16, None, 16, None, 0.0, None) == -1  # hn without gain
for _ in range(1000):  # the thread-local error string, rewritten many times
    lib.spec_kv_set_len(None, 1, None, 1, None)
    assert bd.spec_last_error()
print("SANITIZED-OK")
"""


def _asan_runtime():
    hits = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


@pytest.mark.timeout(600)
def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    from draft_then_verify_amd import build as B

    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    rt = _asan_runtime()
    if not os.path.exists(hipcc) or rt is None:
        pytest.skip("hipcc or the ASan runtime is not available")
    if not os.path.exists(os.path.join(BUILD, "capi.o")):
        B.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
    flags = [f for f in B.COMMON_FLAGS if f != "-O3"] + ["-O1", "-g"]
    obj = str(tmp_path / "capi_san.o")
    r = subprocess.run([hipcc, *flags, *san, "-c", os.path.join(B.CSRC, "capi.hip"), "-o", obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    others = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "capi.hip"]
    lib = str(tmp_path / "libspecverify_san.so")
    r = subprocess.run([hipcc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *san, obj, *others, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    code = f"ROOT = {ROOT!r}\nLIB = {lib!r}\n" + CALLS
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "SANITIZED-OK" in r.stdout, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
