"""The graph-replayed generation (drafter passes + verify step + round
bookkeeping on the device, one HIP graph replay per round) emits exactly the
tokens of the host-driven generation: same models, prompts and per-round
uniforms.  Each replay re-reads the uniforms copied in by the host, so every
round of the graph is checked.  (test_gpu_configs replays graph-generated
rounds through the oracle itself.)  Finished sequences are frozen by the round
bookkeeping: their caches stop growing while the others finish."""
import numpy as np
import pytest

from draft_then_verify_amd import binding as bd
from draft_then_verify_amd.runner import DeviceNgramDrafter, ModelDrafter, SpecDecoder
from synth import SHAPES, make_markov_table, make_prompt, make_weights, markov_prompt
from tests._gpu import to_dev

pytestmark = pytest.mark.gpu


def _sub(w, layers):
    return {k: (v[:layers] if k in ("attn_norm", "wqkv", "wo", "mlp_norm", "wgu", "wd") else v) for k, v in w.items()}


def _pair(shape, B, g, P, N, seed, draft_layers, T=1.0):
    w = make_weights(shape, seed=seed)
    max_ctx = P + N + 2 * g + 4
    prompt = make_prompt(B, P, shape.vocab, seed=seed)
    target = bd.SpecModel(shape, to_dev(w))
    outs = []
    for mode in ("eager", "graph"):
        drafter = None
        if g:
            dsh = shape.with_(n_layers=draft_layers)
            drafter = ModelDrafter(bd.SpecModel(dsh, to_dev(_sub(w, draft_layers))), B, g, max_ctx, temperature=T)
        dec = SpecDecoder(target, B, g, max_ctx, drafter=drafter, temperature=T, seed=seed)
        dec.prefill(prompt)
        res = dec.generate(N) if mode == "eager" else dec.generate_graph(N)
        outs.append(res)
    assert outs[0]["tokens"] == outs[1]["tokens"]
    assert outs[0]["rounds"] <= outs[1]["rounds"] <= outs[0]["rounds"] + 1
    # acceptance counted per sequence until it has its tokens, the same either way
    for k in ("mean_acceptance_length", "acceptance_rate", "per_position"):
        assert outs[0].get(k) == outs[1].get(k), k
    return outs


def test_graph_rounds_tiny_speculative():
    _pair(SHAPES["tiny"], B=1, g=4, P=64, N=32, seed=401, draft_layers=1)


def test_graph_rounds_small_batch():
    _pair(SHAPES["small"], B=3, g=4, P=40, N=48, seed=402, draft_layers=2)


def test_graph_rounds_plain_decoding():
    _pair(SHAPES["small"], B=2, g=0, P=24, N=20, seed=403, draft_layers=0)


def test_greedy_speculation_equals_greedy_decoding():
    """At temperature 0 the speculative output is plain greedy decoding of the
    target, token for token ("How Speculative Decoding Works", section
    "Exactness is a choice"): graph-replayed greedy rounds with a one-layer
    drafter against gamma = 0 greedy decoding of the same float32 target."""
    shape = SHAPES["tiny"]
    spec = _pair(shape, B=2, g=4, P=48, N=40, seed=404, draft_layers=1, T=0.0)
    plain = _pair(shape, B=2, g=0, P=48, N=40, seed=404, draft_layers=0, T=0.0)
    assert spec[1]["tokens"] == plain[0]["tokens"]
    assert spec[1]["rounds"] <= plain[0]["rounds"]


@pytest.mark.parametrize("B,n_min,n_max", [(1, 3, 3), (4, 3, 3), (4, 2, 6)])
def test_graph_rounds_device_ngram_equal_eager(B, n_min, n_max):
    """Prompt lookup on the device inside the replayed rounds (bound once to
    the buffers the rounds append to) proposes what the eager rounds' lookup
    (handed the whole committed context each round) does, so the two
    generations emit the same tokens: the copy-heavy workload's shape
    (trigram lookup or a 2..6 window, gamma = 10, order-2 Markov prompts,
    misses padded from a seeded prompt offset, one-hot q) on the second
    workload's body with a 151936-entry vocabulary, two layers."""
    shape = SHAPES["small_v151936"].with_(n_layers=2)
    w = make_weights(shape, seed=406)
    P, g, N = 256, 10, 48
    max_ctx = P + N + 2 * g + 4
    table = make_markov_table(seed=406)
    prompt = markov_prompt(B, P, table, seed=407).astype(np.int64)
    offs = np.random.default_rng(408).integers(0, P - g - 1, size=B)
    target = bd.SpecModel(shape, to_dev(w))
    outs = []
    for mode in ("eager", "graph"):
        drafter = DeviceNgramDrafter(B, g, n=n_min, n_max=n_max, fill_off=offs)
        dec = SpecDecoder(target, B, g, max_ctx, drafter=drafter, seed=406)
        dec.prefill(prompt)
        outs.append(dec.generate(N) if mode == "eager" else dec.generate_graph(N))
    assert outs[0]["tokens"] == outs[1]["tokens"]
    assert outs[0]["rounds"] <= outs[1]["rounds"] <= outs[0]["rounds"] + 1
    assert 0.0 <= outs[1]["ngram_hit_rate"] <= 1.0


def test_graph_rounds_freeze_finished_sequences():
    """B = 8 sequences finish after different numbers of rounds; a finished
    sequence's later rounds are discarded and its KV length restored, so every
    cache ends within prompt + n_new + gamma positions and the counted rounds
    of each sequence are exactly the rounds it needed."""
    shape = SHAPES["small"].with_(n_layers=2)
    w = make_weights(shape, seed=410)
    B, g, P, N = 8, 4, 32, 40
    max_ctx = P + N + 2 * g + 4
    prompt = make_prompt(B, P, shape.vocab, seed=410)
    target = bd.SpecModel(shape, to_dev(w))
    drafter = ModelDrafter(bd.SpecModel(shape.with_(n_layers=1), to_dev(_sub(w, 1))), B, g, max_ctx)
    dec = SpecDecoder(target, B, g, max_ctx, drafter=drafter, seed=410)
    dec.prefill(prompt)
    res = dec.generate_graph(N)
    lens = dec.kv.len.cpu().numpy()
    assert (lens <= P - 1 + N + g).all()
    assert max(res["sequence_rounds"]) == res["rounds"]
    for b in range(B):
        # the committed context is the prompt plus the emitted tokens; the
        # target cache holds all of it but the last token
        assert lens[b] == len(dec.committed[b]) - 1
        assert len(dec.committed[b]) - P >= N
