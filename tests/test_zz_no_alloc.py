"""spec_decode_step_static (the decode step with the library's own device
workspace, for callers that cannot allocate) against spec_decode_step with a
caller workspace: two steps in a row, the second smaller, each run through
both entry points from the same cache state; integers, logits and committed
lengths bitwise equal.  A step too large for the array is refused."""
import numpy as np
import pytest
import torch

from draft_then_verify_amd import binding as bd
from synth import SHAPES, make_prompt, make_weights, round_uniforms
from tests._gpu import f32, gpu_prefill, gpu_softmax, i32, to_dev

pytestmark = pytest.mark.gpu


def test_static_workspace_matches_caller_workspace():
    shape = SHAPES["small"].with_(n_layers=2)
    w = make_weights(shape, seed=501, norm="random")
    model = bd.SpecModel(shape, to_dev(w))
    V, P, B0 = shape.vocab, 40, 3
    max_ctx = P + 2 * 5 + 8
    kv = bd.KVCache(shape, 2, B0, max_ctx)
    prompt = make_prompt(B0, P, V, seed=501)
    gpu_prefill(model, kv, prompt)
    rng = np.random.default_rng(501)
    last = prompt[:, -1].astype(np.int64)
    for step, (B, g) in enumerate(((3, 4), (2, 2))):  # the second call is smaller
        drafts = rng.integers(0, V, size=(B, g))
        q = gpu_softmax(torch.randn((B * g, V), device="cuda") * 2, V).reshape(B, g, V)
        u = round_uniforms(501, step, B, g)
        len0 = kv.len.clone()
        outs = []
        for static in (False, True):
            kv.len.copy_(len0)
            n = torch.full((B,), -7, dtype=torch.int32, device="cuda")
            em = torch.full((B, g + 1), -7, dtype=torch.int32, device="cuda")
            lo = torch.full((B, g + 1, V), float("nan"), device="cuda")
            args = (model, kv, B, g, 1.0, i32(last[:B]), i32(drafts), None, q, f32(u["u_acc"]), f32(u["u_res"]),
                    n, em, lo)
            if static:
                bd.spec_decode_step_static(*args)
            else:
                bd.spec_decode_step(*args, bd.workspace(model.workspace_bytes(B, g + 1, max_ctx)))
            torch.cuda.synchronize()
            outs.append((n.cpu().numpy(), em.cpu().numpy(), lo.cpu().numpy(), kv.len.cpu().numpy()))
        (n_a, em_a, lo_a, len_a), (n_b, em_b, lo_b, len_b) = outs
        assert np.array_equal(n_a, n_b) and np.array_equal(em_a, em_b) and np.array_equal(len_a, len_b)
        assert np.array_equal(lo_a.view(np.int32), lo_b.view(np.int32))
        assert (n_a >= 0).all() and (n_a <= g).all()
        last = em_b[np.arange(B), n_b]


def test_static_workspace_refuses_oversize_steps():
    shape = SHAPES["small_v151936"].with_(n_layers=1)
    w = make_weights(shape, seed=502)
    model = bd.SpecModel(shape, to_dev(w))
    B, g = 64, 10
    kv = bd.KVCache(shape, 1, B, 64)
    assert model.workspace_bytes(B, g + 1, 64) > bd.load_library().spec_workspace_bytes(model.handle, 1, 5, 64)
    with pytest.raises(bd.SpecError) as e:
        n = torch.empty(B, dtype=torch.int32, device="cuda")
        em = torch.empty((B, g + 1), dtype=torch.int32, device="cuda")
        bd.spec_decode_step_static(model, kv, B, g, 0.0, i32(np.zeros(B)), i32(np.zeros((B, g))), None, None, None,
                                   None, n, em, None)
    assert e.value.status == -4 and "workspace" in str(e.value)
