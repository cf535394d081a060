"""The C ABI library: it loads, exports every symbol the header declares, and
its host-side argument checks reject bad calls before any launch (no GPU)."""
import ctypes
import os
import re

import pytest

from draft_then_verify_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        from draft_then_verify_amd import build
        build.build()
    return bd.load_library()


def header_functions():
    src = open(os.path.join(ROOT, "include", "spec_verify.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) == 16
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(bd.EXPORTS) == names


def test_sampler_workspace_size(lib):
    # 151936 entries -> 38 chunks of 4096; 8 bytes per (row, chunk), 16 per (sequence, chunk)
    assert bd.spec_sampler_workspace_bytes(5, 0, 151936) == 5 * 38 * 8 + (256 - 5 * 38 * 8 % 256) % 256
    assert bd.spec_sampler_workspace_bytes(0, 3, 8) == 256
    assert bd.spec_sampler_workspace_bytes(-1, 0, 8) == 0


def test_host_checks_reject_before_launch(lib):
    cfg = bd.spec_model_cfg(256, 4, 4, 4, 96, 704, 4096, bd.SPEC_F32, 10000.0, 1e-6)
    w = bd.spec_weights()
    h = ctypes.c_void_p()
    assert lib.spec_model_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)) == -4  # head_dim 96
    assert "head_dim" in bd.spec_last_error()
    cfg.head_dim = 64
    assert lib.spec_model_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)) == -1  # NULL weights
    assert lib.spec_model_create(None, None, None) == -1
    # sampler argument checks
    st = lib.spec_reject_sample(0, 4, 100, 1, None, 1, None, 1, 1, 1, 1, 1, 1 << 20, None)
    assert st == -1 and "B=0" in bd.spec_last_error()
    st = lib.spec_reject_sample(1, -1, 100, 1, None, 1, None, 1, 1, 1, 1, 1, 1 << 20, None)
    assert st == -1
    st = lib.spec_reject_sample(1, 2, 1 << 23, 1, None, 1, None, 1, 1, 1, 1, 1, 1 << 20, None)
    assert st == -1
    st = lib.spec_reject_sample(1, 2, 100, 1, None, None, None, 1, 1, 1, 1, 1, 1 << 20, None)
    assert st == -1  # draft NULL with gamma > 0
    st = lib.spec_reject_sample(1, 2, 100, 1, None, 1, None, 1, 1, 1, 1, 1, 8, None)
    assert st == -2  # workspace too small
    for bad_t in (-1.0, float("nan"), float("inf")):  # temperature must be finite and >= 0
        assert lib.spec_softmax_pq(1, 4, 100, bad_t, 1, 1, 1 << 20, None) == -1
    st = lib.spec_reject_sample(1, 2, 100, 1, None, 1, None, None, 1, 1, 1, 1, 1 << 20, None)
    assert st == -1  # u_acc NULL with gamma > 0
    # draft sampling: buffers present, B and vocab in range, strides at least a row, u for T > 0, workspace
    #   spec_draft_sample(logits, ld_logits, B, vocab, T, u, q, ld_q, tokens, ld_tokens, ws, ws_bytes, stream)
    assert lib.spec_draft_sample(None, 100, 1, 100, 1.0, 1, 1, 100, 1, 1, 1, 1 << 20, None) == -1
    assert lib.spec_draft_sample(1, 100, 0, 100, 1.0, 1, 1, 100, 1, 1, 1, 1 << 20, None) == -1  # B = 0
    assert lib.spec_draft_sample(1, 100, 1, 1 << 23, 1.0, 1, 1, 1 << 23, 1, 1, 1, 1 << 30, None) == -1
    assert lib.spec_draft_sample(1, 99, 1, 100, 1.0, 1, 1, 100, 1, 1, 1, 1 << 20, None) == -1  # ld_logits < vocab
    assert lib.spec_draft_sample(1, 100, 2, 100, 1.0, 1, 1, 50, 1, 1, 1, 1 << 20, None) == -1  # ld_q < vocab
    assert lib.spec_draft_sample(1, 100, 2, 100, 1.0, 1, 1, 100, 1, 0, 1, 1 << 20, None) == -1  # ld_tokens 0
    assert lib.spec_draft_sample(1, 100, 1, 100, 1.0, None, 1, 100, 1, 1, 1, 1 << 20, None) == -1  # u NULL, T > 0
    assert lib.spec_draft_sample(1, 100, 1, 100, float("nan"), 1, 1, 100, 1, 1, 1, 1 << 20, None) == -1
    assert lib.spec_draft_sample(1, 100, 4, 100, 1.0, 1, 1, 100, 1, 1, 1, 8, None) == -2  # workspace too small
    assert lib.spec_kv_set_len(None, 1, None, 1, None) == -1
    kv = bd.spec_kv(1, 1, 1, 2, 16)
    assert lib.spec_kv_set_len(ctypes.byref(kv), 3, None, 1, None) == -1
    assert lib.spec_verify_forward(None, ctypes.byref(kv), 1, 1, 1, None, 1, 1 << 30, None) == -1
    assert lib.spec_workspace_bytes(None, 1, 1, 16) == 0
    assert lib.spec_commit_round(0, 4, 1, 1, 1, None, 1, 1, 8, 0, None, None, None, 0, None) == -1
    assert lib.spec_commit_round(1, 4, None, 1, 1, None, 1, 1, 8, 0, None, None, None, 0, None) == -1
    assert lib.spec_commit_round(1, 4, 1, 1, 1, None, 1, 1, 8, -1, None, None, None, 0, None) == -1  # n_stop < 0
    assert lib.spec_commit_round(1, 4, 1, 1, 1, None, 1, 1, 8, 0, None, None, 1, 4, None) == -1  # log, no counts
    assert lib.spec_commit_round(1, 4, 1, 1, 1, None, 1, 1, 8, 0, None, 1, 1, 0, None) == -1  # log_cap 0
    # n-gram lookup: 1 <= n_min <= n_max <= 16, gamma in 0..63, buffers present
    assert lib.spec_ngram_propose(1, 0, 3, 4, 1, None, 8, None, None, 0, None, 1, 1, None, None) == -1
    assert lib.spec_ngram_propose(1, 4, 3, 4, 1, None, 8, None, None, 0, None, 1, 1, None, None) == -1
    assert lib.spec_ngram_propose(1, 3, 17, 4, 1, None, 8, None, None, 0, None, 1, 1, None, None) == -1
    assert lib.spec_ngram_propose(1, 3, 3, 64, 1, None, 8, None, None, 0, None, 1, 1, None, None) == -1
    assert lib.spec_ngram_propose(1, 3, 3, 4, 1, None, 8, 1, None, 4, None, 1, 1, None, None) == -1  # out_len NULL
    assert lib.spec_ngram_propose(1, 3, 3, 4, None, None, 0, 1, 1, 4, 1, 1, 1, None, None) == -1   # fill, no prefix


def test_missing_library_fails_loudly(tmp_path):
    """Without the built library the binding raises (there is no fallback
    path); run in a fresh interpreter, since a loaded library is cached."""
    import subprocess
    import sys

    missing = str(tmp_path / "libspecverify.so")
    code = ("from draft_then_verify_amd import binding as bd\n"
            f"bd.load_library({missing!r})\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=str(__import__("pathlib").Path(__file__).resolve().parents[1]))
    assert r.returncode != 0
    assert "is missing" in r.stderr and "no fallback" in r.stderr


def test_check_mode_keeps_the_argument_checks(tmp_path):
    """With SPEC_CHECK=1 the host-side argument checks still come first: bad
    arguments are SPEC_EINVAL / SPEC_ENOMEM, never a validation result."""
    import subprocess
    import sys

    code = ("import ctypes\nfrom draft_then_verify_amd import binding as bd\nlib = bd.load_library()\n"
            "assert lib.spec_reject_sample(0, 4, 100, 1, None, 1, None, 1, 1, 1, 1, 1, 1 << 20, None) == -1\n"
            "assert lib.spec_reject_sample(1, 2, 100, 1, None, 1, None, 1, 1, 1, 1, 1, 8, None) == -2\n"
            "assert lib.spec_softmax_pq(None, 4, 100, 1.0, 1, 1, 1 << 20, None) == -1\n"
            "kv = bd.spec_kv(1, 1, 1, 2, 16)\n"
            "assert lib.spec_verify_forward(None, ctypes.byref(kv), 1, 1, 1, None, 1, 1 << 30, None) == -1\n"
            "print('ok')\n")
    env = dict(os.environ, SPEC_CHECK="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT)
    assert r.returncode == 0 and "ok" in r.stdout, r.stderr[-2000:]
