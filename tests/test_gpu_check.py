"""Validation mode (SPEC_CHECK=1): token ids outside [0, vocab) and
non-finite logits or probability rows make the call return SPEC_EDEVICE
after the stream is synchronised; valid inputs give the same results as
without the mode."""
import numpy as np
import pytest
import torch

from draft_then_verify_amd import binding as bd
from synth import SHAPES, make_prompt, make_weights, round_uniforms
from tests._gpu import f32, gpu_prefill, gpu_softmax, i32, to_dev

pytestmark = pytest.mark.gpu


def _setup(seed=601, poison_row=None):
    shape = SHAPES["small"].with_(n_layers=1)
    w = make_weights(shape, seed=seed)
    if poison_row is not None:
        w["lm_head"] = w["lm_head"].clone()
        w["lm_head"][poison_row] = float("inf")
    model = bd.SpecModel(shape, to_dev(w))
    B, g, P = 2, 4, 16
    max_ctx = P + 12
    kv = bd.KVCache(shape, 1, B, max_ctx)
    prompt = make_prompt(B, P, shape.vocab, seed=seed)
    gpu_prefill(model, kv, prompt)
    return shape, model, kv, prompt, B, g, max_ctx


def _step(model, kv, prompt, B, g, max_ctx, drafts, V, lo=None):
    u = round_uniforms(601, 0, B, g)
    q = gpu_softmax(torch.randn((B * g, V), device="cuda"), V).reshape(B, g, V)
    n = torch.empty(B, dtype=torch.int32, device="cuda")
    em = torch.empty((B, g + 1), dtype=torch.int32, device="cuda")
    bd.spec_decode_step(model, kv, B, g, 1.0, i32(prompt[:, -1]), i32(drafts), None, q, f32(u["u_acc"]),
                        f32(u["u_res"]), n, em, lo, bd.workspace(model.workspace_bytes(B, g + 1, max_ctx)))
    torch.cuda.synchronize()
    return n.cpu().numpy(), em.cpu().numpy()


def test_check_mode_same_results_on_valid_inputs(monkeypatch):
    shape, model, kv, prompt, B, g, max_ctx = _setup()
    V = shape.vocab
    drafts = np.random.default_rng(1).integers(0, V, size=(B, g))
    len0 = kv.len.clone()
    torch.manual_seed(0)
    a = _step(model, kv, prompt, B, g, max_ctx, drafts, V)
    kv.len.copy_(len0)
    monkeypatch.setenv("SPEC_CHECK", "1")
    torch.manual_seed(0)
    b = _step(model, kv, prompt, B, g, max_ctx, drafts, V)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_check_mode_rejects_out_of_range_draft(monkeypatch):
    shape, model, kv, prompt, B, g, max_ctx = _setup()
    V = shape.vocab
    drafts = np.random.default_rng(2).integers(0, V, size=(B, g))
    drafts[1, 2] = V
    monkeypatch.setenv("SPEC_CHECK", "1")
    with pytest.raises(bd.SpecError) as e:
        _step(model, kv, prompt, B, g, max_ctx, drafts, V)
    assert e.value.status == -5 and "token id" in str(e.value)


def test_check_mode_rejects_non_finite_logits(monkeypatch):
    shape, model, kv, prompt, B, g, max_ctx = _setup(poison_row=7)
    V = shape.vocab
    drafts = np.random.default_rng(3).integers(0, V, size=(B, g))
    monkeypatch.setenv("SPEC_CHECK", "1")
    with pytest.raises(bd.SpecError) as e:
        _step(model, kv, prompt, B, g, max_ctx, drafts, V)
    assert e.value.status == -5 and "non-finite" in str(e.value)


def test_check_mode_sampler_rows(monkeypatch):
    """spec_reject_sample: a NaN in p, and a draft id of -1, are reported."""
    B, g, V = 3, 2, 1000
    p = gpu_softmax(torch.randn((B * (g + 1), V), device="cuda"), V).reshape(B, g + 1, V).contiguous()
    drafts = i32(np.zeros((B, g)))
    u = f32(np.full((B, g), 0.5))
    ur = f32(np.full(B, 0.5))
    n = torch.empty(B, dtype=torch.int32, device="cuda")
    em = torch.empty((B, g + 1), dtype=torch.int32, device="cuda")
    ws = bd.workspace(bd.spec_sampler_workspace_bytes(0, B, V))
    monkeypatch.setenv("SPEC_CHECK", "1")
    bd.spec_reject_sample(B, g, V, p, None, drafts, None, u, ur, n, em, ws)
    p[1, 0, 5] = float("nan")
    with pytest.raises(bd.SpecError) as e:
        bd.spec_reject_sample(B, g, V, p, None, drafts, None, u, ur, n, em, ws)
    assert e.value.status == -5
    p[1, 0, 5] = 0.0
    drafts[2, 1] = -1
    with pytest.raises(bd.SpecError) as e:
        bd.spec_reject_sample(B, g, V, p, None, drafts, None, u, ur, n, em, ws)
    assert e.value.status == -5 and "token id" in str(e.value)
