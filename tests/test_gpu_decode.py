"""GPU parity of the fused decode step (verify pass + softmax + accept /
resample / bonus + KV commit) against the oracle's round, teacher-forced:
both sides get the same drafts, draft rows and uniforms."""
import numpy as np
import pytest
import torch

from draft_then_verify_amd import binding as bd
from oracle import model as OM
from oracle import rounds as R
from oracle import sampler as S
from synth import SHAPES, make_prompt, make_weights, round_uniforms
from tests._gpu import f32, gpu_prefill, gpu_softmax, i32, to_dev

pytestmark = pytest.mark.gpu


def _decode_round(shape, B, g, seed, onehot=False, ragged=False, n_layers=None, P=48):
    w = make_weights(shape, seed=seed, norm="random", layers=n_layers)
    sh = shape if n_layers is None else shape.with_(n_layers=n_layers)
    max_ctx = P + g + 4
    model = bd.SpecModel(sh, to_dev(w))
    kv = bd.KVCache(sh, sh.n_layers, B, max_ctx)
    prompt = make_prompt(B, P, sh.vocab, seed=seed)
    gpu_prefill(model, kv, prompt)
    tgt = OM.Decoder(sh, w)
    ct = tgt.new_cache(B, max_ctx)
    R.prefill(tgt, ct, prompt)
    # drafts from a one-layer drafter of the oracle (teacher-forced inputs)
    u = round_uniforms(seed, 0, B, g)
    if onehot:
        rng = np.random.default_rng(seed)
        drafts, q = rng.integers(0, sh.vocab, size=(B, g)), None
    else:
        dft = OM.Decoder(sh, w, n_layers=1)
        cd = dft.new_cache(B, max_ctx)
        R.prefill(dft, cd, prompt)
        drafts, q = R.draft_round(dft, cd, prompt[:, -2], prompt[:, -1], ct.length, g, u["u_draft"])
    nd = np.random.default_rng(seed + 1).integers(0, g + 1, size=B) if ragged else None
    n_g = torch.empty(B, dtype=torch.int32, device="cuda")
    em_g = torch.empty((B, g + 1), dtype=torch.int32, device="cuda")
    logits = torch.empty((B, g + 1, sh.vocab), dtype=torch.float32, device="cuda")
    ws = bd.workspace(model.workspace_bytes(B, g + 1, max_ctx))
    len0 = kv.len.clone()
    bd.spec_decode_step(model, kv, B, g, 1.0, i32(prompt[:, -1]), i32(drafts), None if nd is None else i32(nd),
                        None if q is None else f32(q), f32(u["u_acc"]), f32(u["u_res"]), n_g, em_g, logits, ws)
    torch.cuda.synchronize()
    out = R.verify_round(tgt, ct, prompt[:, -1], drafts, q, nd, u["u_acc"], u["u_res"])
    n_g, em_g = n_g.cpu().numpy(), em_g.cpu().numpy()
    # logits parity
    tol = 1e-4 if sh.dtype == "f32" else 2e-2
    assert np.abs(logits.cpu().numpy() - out["logits"]).max() < tol
    # the GPU's own p rows, sampled by the oracle's rule, give exactly the GPU's integers
    p_gpu = gpu_softmax(logits, sh.vocab).cpu().numpy()
    assert np.abs(p_gpu - out["p"]).max() < 1e-5
    n_o, em_o = S.reject_sample(p_gpu, q, drafts, nd, u["u_acc"], u["u_res"])
    assert np.array_equal(n_g, n_o) and np.array_equal(em_g, em_o)
    # against the oracle's own p: identical except decisions within 1e-4 of the threshold
    qx = np.ones((B, g)) if q is None else np.take_along_axis(q, drafts[:, :, None], 2)[..., 0]
    px = np.take_along_axis(out["p"][:, :g], drafts[:, :, None], 2)[..., 0]
    near = np.abs(u["u_acc"] - np.minimum(1.0, px / np.maximum(qx, 1e-30))) < 1e-4
    same = n_g == out["n"]
    assert (same | near.any(axis=1)).all()
    # KV commit
    assert np.array_equal(kv.len.cpu().numpy(), len0.cpu().numpy() + n_g + 1)
    return n_g, em_g


def test_decode_step_tiny_f32():
    _decode_round(SHAPES["tiny"], B=1, g=4, seed=201)


def test_decode_step_small_bf16_batch():
    _decode_round(SHAPES["small"], B=4, g=4, seed=202, n_layers=2)


def test_decode_step_onehot_ragged_v151936():
    """Long one-hot draft (n-gram style) with ragged n_draft over a
    151936-entry vocabulary."""
    shape = SHAPES["small_v151936"]
    _decode_round(shape, B=3, g=10, seed=203, onehot=True, ragged=True, n_layers=1, P=24)
