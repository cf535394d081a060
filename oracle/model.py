"""Oracle decoder forward pass (test infrastructure; see package docstring).

What a verify pass computes [P1 "What one iteration actually does", Algorithm 1,
the parallel scoring step; P3 "How speculative decoding works"]: the target
scores every drafted position in one forward pass, row i being the next-token
distribution after the prefix plus the first i inputs.  The pages name no
architecture beyond "Llama-style"/"Qwen3-8B-shaped", so the plainest Llama
reading is taken: pre-norm RMSNorm (eps 1e-6), rotate-half RoPE (theta
10000), grouped-query attention (query head h reads KV head h // (H / Hkv)),
SwiGLU MLP, no biases, no QK-norm, untied head unless the shape says tied.

Precision contract for bf16 models: every linear input is rounded to bf16,
K/V are stored as bf16, everything else is exact fp64 here (fp32 on the GPU).
For f32 models nothing is rounded.  Written for clarity, not speed: one
matmul per linear, one loop iteration per (sequence, row) in attention.
"""

from __future__ import annotations

import numpy as np

from .bf16 import round_bf16


def _np(t) -> np.ndarray:
    """Weights arrive as torch tensors (float32/bfloat16) or numpy arrays;
    keep them as float32 arrays holding the exact values."""
    if isinstance(t, np.ndarray):
        return t
    import torch  # plain tensor -> array conversion only

    return t.detach().to("cpu", torch.float32).numpy()


def rms_norm(h: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """h / sqrt(mean(h^2) + eps) * g over the last axis."""
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps) * g


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding.  x [..., n_heads, hd], pos broadcastable
    to x.shape[:-2].  Pair (i, i + hd/2) is rotated by angle pos * theta^(-2i/hd)."""
    hd = x.shape[-1]
    half = hd // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / hd)
    ang = np.asarray(pos, dtype=np.float64)[..., None, None] * inv_freq  # [..., 1, half]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Grouped-query attention of one query row over n keys.

    q [H, hd]; K, V [Hkv, n, hd].  Query head h reads KV head h // (H / Hkv);
    scores are q.k / sqrt(hd), softmax over the n keys, output the weighted
    sum of V rows.  Returns [H, hd]."""
    H, hd = q.shape
    Hkv = K.shape[0]
    G = H // Hkv
    qh = q.reshape(Hkv, G, hd)
    sc = np.einsum("kgd,knd->kgn", qh, K) / np.sqrt(hd)
    sc = sc - sc.max(axis=-1, keepdims=True)
    e = np.exp(sc)
    pr = e / e.sum(axis=-1, keepdims=True)
    return np.einsum("kgn,knd->kgd", pr, V).reshape(H, hd)


def linear(x: np.ndarray, W: np.ndarray, bf16: bool) -> np.ndarray:
    """y = x W^T in fp64; under the bf16 contract the input x is first rounded
    to bf16 (W already holds bf16 values)."""
    if bf16:
        x = round_bf16(x)
    return x @ np.asarray(W, dtype=np.float64).T


class KVCache:
    """Per-sequence contiguous cache: k, v [L, B, Hkv, max_ctx, hd] and the
    committed length per sequence.  A forward pass writes rows at
    length[b] .. length[b] + m - 1 and leaves ``length`` unchanged."""

    def __init__(self, n_layers, B, n_kv_heads, max_ctx, head_dim):
        self.k = np.zeros((n_layers, B, n_kv_heads, max_ctx, head_dim), dtype=np.float64)
        self.v = np.zeros_like(self.k)
        self.length = np.zeros(B, dtype=np.int64)
        self.max_ctx = max_ctx


class Decoder:
    """Llama-style decoder over given weights (dict as produced by synth.make_weights).

    ``n_layers`` < shape.n_layers runs only the first layers, then the final
    norm and the head: the self-speculative drafter [P5 "What it looks like in
    code", the simpler variant that drafts with the target's own early layers].
    """

    def __init__(self, shape, weights: dict, n_layers: int | None = None, precast: bool = False):
        """``precast`` stores the weight matrices as float64 once instead of
        widening them at every matmul: the same arithmetic, traded for memory
        (used at the 8B shape, where the per-call widening dominates)."""
        self.shape = shape
        self.L = shape.n_layers if n_layers is None else n_layers
        self.bf16 = shape.dtype == "bf16"
        self.w = {}
        for k, v in weights.items():
            a = _np(v)
            if precast and a.ndim >= 2:
                if k in ("attn_norm", "wqkv", "wo", "mlp_norm", "wgu", "wd"):
                    a = a[: self.L]
                a = a.astype(np.float64)
            self.w[k] = a

    def new_cache(self, B: int, max_ctx: int) -> KVCache:
        s = self.shape
        return KVCache(self.L, B, s.n_kv_heads, max_ctx, s.head_dim)

    def layer_weights(self, layer: int) -> dict:
        """The weights of one layer (attn_norm, wqkv, wo, mlp_norm, wgu, wd)."""
        return {k: self.w[k][layer] for k in ("attn_norm", "wqkv", "wo", "mlp_norm", "wgu", "wd")}

    def forward(self, cache: KVCache, tokens: np.ndarray, logits: bool = True):
        """tokens [B, m] int -> logits [B, m, V] fp64 (None when ``logits`` is
        False, as in prefill); writes K/V at the m new positions."""
        s, w = self.shape, self.w
        tokens = np.asarray(tokens)
        B, m = tokens.shape
        pos = cache.length[:, None] + np.arange(m)[None, :]  # [B, m]
        if int(pos.max()) >= cache.max_ctx:
            raise ValueError("KV cache too short for this pass")
        h = w["embed"][tokens].astype(np.float64)  # [B, m, d]
        for layer in range(self.L):
            h = decoder_layer(s, self.layer_weights(layer), h, cache.k[layer], cache.v[layer], pos, self.bf16)
        if not logits:
            return None
        return final_logits(s, w["final_norm"], w["lm_head"], h, self.bf16)


def decoder_layer(s, lw: dict, h: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, pos: np.ndarray,
                  bf16: bool) -> np.ndarray:
    """One pre-norm decoder layer over residual rows h [B, m, d] at positions
    pos [B, m]: attention block then MLP block, each added to the residual.
    k_cache, v_cache [B, Hkv, max_ctx, hd] are this layer's cache; the new
    rows are written at pos and row (b, i) attends to keys 0 .. pos[b, i].
    Returns the new residual rows (fp64)."""
    B, m = pos.shape
    H, Hkv, hd, F = s.n_heads, s.n_kv_heads, s.head_dim, s.d_ff
    store = round_bf16 if bf16 else (lambda x: x)
    a = rms_norm(h, np.asarray(lw["attn_norm"], np.float64), s.rms_eps)
    qkv = linear(a, lw["wqkv"], bf16)
    q = qkv[..., : H * hd].reshape(B, m, H, hd)
    k = qkv[..., H * hd: (H + Hkv) * hd].reshape(B, m, Hkv, hd)
    v = qkv[..., (H + Hkv) * hd:].reshape(B, m, Hkv, hd)
    q = rope(q, pos, s.rope_theta)
    k = rope(k, pos, s.rope_theta)
    bidx = np.repeat(np.arange(B), m)
    k_cache[bidx, :, pos.reshape(-1)] = store(k.reshape(B * m, Hkv, hd))
    v_cache[bidx, :, pos.reshape(-1)] = store(v.reshape(B * m, Hkv, hd))
    o = np.zeros((B, m, H, hd))
    for b in range(B):
        for i in range(m):
            n_keys = pos[b, i] + 1  # causal: keys 0 .. pos
            o[b, i] = attend(q[b, i], k_cache[b, :, :n_keys], v_cache[b, :, :n_keys])
    h = h + linear(o.reshape(B, m, H * hd), lw["wo"], bf16)
    a2 = rms_norm(h, np.asarray(lw["mlp_norm"], np.float64), s.rms_eps)
    gu = linear(a2, lw["wgu"], bf16)
    z = silu(gu[..., :F]) * gu[..., F:]
    return h + linear(z, lw["wd"], bf16)


def final_logits(s, final_norm, lm_head, h: np.ndarray, bf16: bool) -> np.ndarray:
    """logits = RMSNorm(h) . W_lm^T (the input rounded to bf16 under the bf16 contract)."""
    a = rms_norm(h, np.asarray(final_norm, np.float64), s.rms_eps)
    return linear(a, lm_head, bf16)
