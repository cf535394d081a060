"""The step-by-step checker of tests/_layerwise.py, pinned on the CPU with a
float32 transcription of one 8B-shape layer (d_model 4096, 32/8 heads,
head_dim 128, d_ff 12288, bf16 weights) as the implementation under test:

* whole layers: the float32 transcription ends the layer measurably apart
  from the fp64 oracle (the bf16 rounding points of the norm and SwiGLU
  outputs turn float32 rounding into one-spacing flips), which is why the
  GPU passes are held step by step;
* every step of the transcription passes the checker at the 2e-2 bar;
* mistakes planted in the transcription (a flipped RoPE sign, a dropped MLP
  norm gain, a query head reading the wrong KV head, a stale residual) fail
  the checker."""
import numpy as np
import pytest
import torch

from oracle import model as OM
from oracle.bf16 import round_bf16
from synth import SHAPES
from tests._layerwise import PassRecord, check_pass

SH = SHAPES["qwen3_8b"].with_(n_layers=1)


@pytest.fixture(scope="module")
def layer():
    s = SH
    g = torch.Generator().manual_seed(0)
    bf = lambda *shape: (torch.randn(*shape, generator=g) * 0.02).to(torch.bfloat16).double().numpy()
    lw = {"attn_norm": 1 + 0.1 * torch.randn(s.d_model, generator=g).double().numpy(),
          "mlp_norm": 1 + 0.1 * torch.randn(s.d_model, generator=g).double().numpy(),
          "wqkv": bf(s.qkv_rows, s.d_model), "wo": bf(s.d_model, s.n_heads * s.head_dim),
          "wgu": bf(2 * s.d_ff, s.d_model), "wd": bf(s.d_model, s.d_ff)}
    h0 = bf(16, s.d_model)
    return lw, h0


def transcribe(lw, h0, plant=None):
    """One layer in float32 arithmetic with the contract's bf16 rounding
    points; returns the trace and the cache it wrote (positions 0..15)."""
    s = SH
    f = np.float32
    H, Hkv, hd, F, d = s.n_heads, s.n_kv_heads, s.head_dim, s.d_ff, s.d_model
    P = h0.shape[0]
    W = {k: v.astype(f) for k, v in lw.items()}

    def rms(h, gain):
        ms = np.mean(h * h, axis=-1, keepdims=True, dtype=f)
        return (h / np.sqrt(ms + f(s.rms_eps)) * gain).astype(f)

    def lin(x, w):
        return (round_bf16(x).astype(f) @ w.T).astype(f)

    def rope(x, pos, sign=1.0):
        half = hd // 2
        ang = pos[:, None, None].astype(np.float64) * (s.rope_theta ** (-(2.0 * np.arange(half)) / hd))
        c, sn = np.cos(ang).astype(f), (sign * np.sin(ang)).astype(f)
        x1, x2 = x[..., :half], x[..., half:]
        return np.concatenate([x1 * c - x2 * sn, x2 * c + x1 * sn], axis=-1).astype(f)

    pos = np.arange(P)
    h = h0.astype(f)
    qkv = lin(rms(h, W["attn_norm"]), W["wqkv"])
    q = rope(qkv[:, :H * hd].reshape(P, H, hd), pos, -1.0 if plant == "rope" else 1.0)
    k = rope(qkv[:, H * hd:(H + Hkv) * hd].reshape(P, Hkv, hd), pos)
    v = qkv[:, (H + Hkv) * hd:].reshape(P, Hkv, hd)
    K = round_bf16(k.transpose(1, 0, 2)).astype(f)
    V = round_bf16(v.transpose(1, 0, 2)).astype(f)
    o = np.zeros((P, H, hd), f)
    G = H // Hkv
    for i in range(P):
        for hh in range(H):
            kh = (hh + 1) % Hkv if plant == "gqa" else hh // G
            sc = (K[kh, :i + 1] @ q[i, hh]) / f(np.sqrt(hd))
            e = np.exp(sc - sc.max())
            o[i, hh] = (e / e.sum()) @ V[kh, :i + 1]
    attn = round_bf16(o.reshape(P, H * hd))
    h_mid = (h + lin(attn, W["wo"])).astype(f)
    gain2 = np.ones(d, f) if plant == "gain" else W["mlp_norm"]
    gu = lin(rms(h_mid, gain2), W["wgu"])
    z = round_bf16(gu[:, :F] / (1 + np.exp(-gu[:, :F])) * gu[:, F:])
    h_out = ((h if plant == "stale" else h_mid) + lin(z, W["wd"])).astype(f)
    trace = {"h": np.stack([h, h_out]).astype(np.float64), "q": q.reshape(1, P, H * hd).astype(np.float64),
             "attn": attn.reshape(1, P, H * hd).astype(np.float64), "h_mid": h_mid[None].astype(np.float64),
             "mlp": z[None].astype(np.float64)}
    return PassRecord("float32 transcription", 1, P, np.zeros(1, np.int64), trace, None,
                      K[None, None].astype(np.float64), V[None, None].astype(np.float64))


def _check(lw, rec):
    return check_pass(SH, lambda layer: lw, None, rec, 2e-2, log=print)


def test_whole_layer_differs_but_every_step_holds(layer):
    lw, h0 = layer
    rec = transcribe(lw, h0)
    # the fp64 oracle's own layer on the same input rows
    kc = np.zeros((1, SH.n_kv_heads, 16, SH.head_dim))
    vc = np.zeros_like(kc)
    ref = OM.decoder_layer(SH, lw, h0[None], kc, vc, np.arange(16)[None], True)[0]
    whole = np.abs(rec.trace["h"][1] - ref).max()
    print(f"whole layer: |float32 - oracle| max {whole:.4f}")
    assert whole > 1e-3  # far above float32 accumulation error: the rounding points flip
    worst = _check(lw, rec)["worst"]
    assert worst["h"] < 1e-3 and worst["h_mid"] < 1e-3  # the linears on identical inputs


@pytest.mark.parametrize("plant", ["rope", "gain", "gqa", "stale"])
def test_planted_mistakes_fail(layer, plant):
    lw, h0 = layer
    with pytest.raises(AssertionError):
        _check(lw, transcribe(lw, h0, plant))
