"""Seeded generators for every synthetic input (weights, prompts, uniforms).

Streams are keyed by (master seed, purpose, index) through numpy's
SeedSequence, so any one tensor or round can be regenerated on its own.

* Weights use torch generators on the device they are created on (fast at the
  8B shape).  A given (seed, device type) always yields the same tensor; tests
  that need the same weights on CPU and GPU create them once and copy.
* Prompts, uniforms and the Markov chain use numpy PCG64 and are identical on
  every machine.
* Uniforms are u = k / 2**24 with k an integer in [0, 2**24): exactly
  representable in float32, so the host and the device see the same value.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch

MASTER_SEED = 20261202

# purpose codes for substreams
_P_WEIGHT = 1
_P_PROMPT = 2
_P_UNIFORM = 3
_P_MARKOV = 4
_P_NORM = 5


@dataclass(frozen=True)
class Shape:
    """Decoder shape (Llama-style: pre-norm RMSNorm, RoPE, SwiGLU, no biases)."""

    name: str
    d_model: int
    n_layers: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    dtype: str  # "f32" or "bf16"
    tied: bool = False  # LM head shares the embedding table
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6

    @property
    def qkv_rows(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    def with_(self, **kw) -> "Shape":
        return replace(self, **kw)

    def param_count(self) -> int:
        d, L, F, V = self.d_model, self.n_layers, self.d_ff, self.vocab
        per_layer = self.qkv_rows * d + d * self.n_heads * self.head_dim + 3 * F * d + 2 * d
        head = 0 if self.tied else V * d
        return V * d + head + L * per_layer + d

    def kv_bytes_per_token(self) -> int:
        b = 4 if self.dtype == "f32" else 2
        return 2 * self.n_layers * self.n_kv_heads * self.head_dim * b


SHAPES = {
    # decoder shapes of the five workloads (target and draft models)
    "tiny": Shape("tiny", 256, 4, 4, 4, 64, 704, 4096, "f32"),
    "small": Shape("small", 1024, 8, 16, 4, 64, 2816, 32000, "bf16"),
    "qwen3_8b": Shape("qwen3_8b", 4096, 36, 32, 8, 128, 12288, 151936, "bf16"),
    "qwen3_0p6b": Shape("qwen3_0p6b", 1024, 28, 16, 8, 128, 3072, 151936, "bf16", tied=True),
    "small_v151936": Shape("small_v151936", 1024, 8, 16, 4, 64, 2816, 151936, "bf16"),
}


def substream_seed(*keys: int) -> int:
    """64-bit seed for the substream named by integer keys."""
    ss = np.random.SeedSequence([int(k) & 0xFFFFFFFF for k in keys])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


def _randn(shape, seed: int, device, std: float) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


_TENSORS = ("wqkv", "wo", "wgu", "wd")


def make_weights(shape: Shape, seed: int = MASTER_SEED, device="cpu", norm: str = "ones",
                 std: float = 0.02, layers: int | None = None) -> dict:
    """Random-init weights, N(0, std) rounded to the model dtype.

    Returns a dict of torch tensors in the row-major [out, in] layout:
      embed [V, d], lm_head [V, d] (the same tensor when tied), final_norm [d],
      attn_norm [L, d], wqkv [L, (H + 2 Hkv) hd, d] (q rows, then k, then v),
      wo [L, d, H hd], mlp_norm [L, d], wgu [L, 2F, d] (gate rows, then up rows),
      wd [L, d, F].
    Norm gains are float32: all ones (``norm="ones"``) or 1 + N(0, 0.1)
    (``norm="random"``, used by tests so that a dropped gain is visible).
    ``layers`` generates only the first layers (the per-layer streams do not
    depend on it).
    """
    dt = torch.float32 if shape.dtype == "f32" else torch.bfloat16
    d, F, V = shape.d_model, shape.d_ff, shape.vocab
    L = shape.n_layers if layers is None else layers
    hq = shape.n_heads * shape.head_dim
    dims = {"wqkv": (shape.qkv_rows, d), "wo": (d, hq), "wgu": (2 * F, d), "wd": (d, F)}
    out: dict = {}
    out["embed"] = _randn((V, d), substream_seed(seed, _P_WEIGHT, 0, 0), device, std).to(dt)
    if shape.tied:
        out["lm_head"] = out["embed"]
    else:
        out["lm_head"] = _randn((V, d), substream_seed(seed, _P_WEIGHT, 1, 0), device, std).to(dt)
    for ti, name in enumerate(_TENSORS):
        t = torch.empty((L,) + dims[name], dtype=dt, device=device)
        for layer in range(L):
            t[layer] = _randn(dims[name], substream_seed(seed, _P_WEIGHT, 10 + ti, layer), device, std).to(dt)
        out[name] = t

    def gains(code, n):
        if norm == "ones":
            return torch.ones(n, dtype=torch.float32, device=device)
        return 1.0 + _randn((n,), substream_seed(seed, _P_NORM, code, 0), device, 0.1)

    out["attn_norm"] = gains(1, L * d).reshape(L, d)
    out["mlp_norm"] = gains(2, L * d).reshape(L, d)
    out["final_norm"] = gains(3, d)
    return out


def make_prompt(B: int, P: int, vocab: int, seed: int = MASTER_SEED, lo: int = 0) -> np.ndarray:
    """[B, P] int32 token ids, uniform in [lo, vocab)."""
    rng = np.random.Generator(np.random.PCG64(substream_seed(seed, _P_PROMPT, B, P)))
    return rng.integers(lo, vocab, size=(B, P), dtype=np.int64).astype(np.int32)


def make_uniforms(shape, seed: int, *keys: int) -> np.ndarray:
    """float32 uniforms k / 2**24, k uniform on [0, 2**24), from substream (seed, keys)."""
    rng = np.random.Generator(np.random.PCG64(substream_seed(seed, _P_UNIFORM, *keys)))
    k = rng.integers(0, 1 << 24, size=shape, dtype=np.int64)
    return (k.astype(np.float64) / float(1 << 24)).astype(np.float32)


def round_uniforms(seed: int, round_idx: int, B: int, gamma: int) -> dict:
    """The uniforms one round consumes: accept tests, the resample/bonus draw,
    and the draft's own sampling, each [B, gamma] or [B]."""
    return {
        "u_acc": make_uniforms((B, max(gamma, 0)), seed, 1, round_idx),
        "u_res": make_uniforms((B,), seed, 2, round_idx),
        "u_draft": make_uniforms((B, max(gamma, 0)), seed, 3, round_idx),
    }


def make_markov_table(seed: int = MASTER_SEED, n_ids: int = 512, n_succ: int = 4):
    """Order-2 Markov chain over ``n_ids`` token ids: each pair (a, b) has
    ``n_succ`` successor ids with Dirichlet(1) weights.  Returns
    (succ [n, n, n_succ] int32, cumw [n, n, n_succ] float64)."""
    rng = np.random.Generator(np.random.PCG64(substream_seed(seed, _P_MARKOV, n_ids, n_succ)))
    succ = rng.integers(0, n_ids, size=(n_ids, n_ids, n_succ), dtype=np.int64).astype(np.int32)
    w = rng.dirichlet(np.ones(n_succ), size=(n_ids, n_ids))
    cumw = np.cumsum(w, axis=-1)
    cumw[..., -1] = 1.0
    return succ, cumw


def markov_prompt(B: int, P: int, table, seed: int = MASTER_SEED) -> np.ndarray:
    """[B, P] int32 prompts walked from the order-2 chain ``table``."""
    succ, cumw = table
    n = succ.shape[0]
    rng = np.random.Generator(np.random.PCG64(substream_seed(seed, _P_MARKOV, B, P, 7)))
    out = np.zeros((B, P), dtype=np.int32)
    out[:, 0] = rng.integers(0, n, size=B)
    if P > 1:
        out[:, 1] = rng.integers(0, n, size=B)
    rows = np.arange(B)
    for t in range(2, P):
        a, b = out[:, t - 2], out[:, t - 1]
        r = rng.random(B)
        idx = (cumw[a, b] <= r[:, None]).sum(axis=1)
        idx = np.minimum(idx, succ.shape[2] - 1)
        out[:, t] = succ[a, b][rows, idx]
    return out
