"""The seeded generators are deterministic and independent per substream."""
import numpy as np
import torch

from synth import SHAPES, make_markov_table, make_prompt, make_uniforms, make_weights, markov_prompt, round_uniforms


def test_weights_deterministic_and_layer_independent():
    s = SHAPES["tiny"].with_(n_layers=3, vocab=256)
    a, b = make_weights(s, seed=1), make_weights(s, seed=1)
    for k in a:
        assert torch.equal(a[k], b[k])
    c = make_weights(s, seed=1, layers=2)
    assert torch.equal(c["wqkv"], a["wqkv"][:2])
    assert not torch.equal(make_weights(s, seed=2)["wqkv"], a["wqkv"])
    bf = make_weights(s.with_(dtype="bf16"), seed=1)
    assert bf["wqkv"].dtype == torch.bfloat16 and bf["final_norm"].dtype == torch.float32
    assert abs(float(a["wqkv"].std()) - 0.02) < 0.001


def test_uniforms_are_exact_grid_values():
    u = make_uniforms((1000,), 3, 1)
    assert u.dtype == np.float32 and (u >= 0).all() and (u < 1).all()
    k = u.astype(np.float64) * (1 << 24)
    assert np.array_equal(k, np.floor(k))
    r = round_uniforms(3, 5, 2, 4)
    assert r["u_acc"].shape == (2, 4) and r["u_res"].shape == (2,)
    assert not np.array_equal(round_uniforms(3, 6, 2, 4)["u_acc"], r["u_acc"])


def test_prompts_and_markov_chain():
    p = make_prompt(3, 50, 100, seed=4)
    assert p.dtype == np.int32 and p.min() >= 0 and p.max() < 100
    assert np.array_equal(p, make_prompt(3, 50, 100, seed=4))
    tab = make_markov_table(seed=4)
    m = markov_prompt(2, 400, tab, seed=4)
    succ, _ = tab
    assert m.max() < 512
    for b in range(2):
        for t in range(2, 400):
            assert m[b, t] in succ[m[b, t - 2], m[b, t - 1]]
