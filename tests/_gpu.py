"""Helpers shared by the GPU parity tests (device plumbing only)."""
import numpy as np
import torch

from draft_then_verify_amd import binding as bd


def to_dev(w: dict) -> dict:
    out = {}
    for k, v in w.items():
        out[k] = v.cuda()
    if w["lm_head"] is w["embed"]:
        out["lm_head"] = out["embed"]
    return out


def i32(a) -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def f32(a) -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def gpu_prefill(model, kv, prompt):
    """K/V for prompt[:, :-1] through the library; len advanced."""
    B, P = prompt.shape
    ws = bd.workspace(model.workspace_bytes(B, P - 1, kv.max_ctx))
    bd.spec_verify_forward(model, kv, B, P - 1, i32(prompt[:, :-1]), None, ws)
    bd.spec_kv_set_len(kv, B, None, P - 1)


def gpu_softmax(logits: torch.Tensor, V: int, T: float = 1.0) -> torch.Tensor:
    rows = logits.numel() // V
    probs = torch.empty_like(logits)
    ws = bd.workspace(bd.spec_sampler_workspace_bytes(rows, 0, V))
    bd.spec_softmax_pq(logits, rows, V, T, probs, ws)
    return probs
