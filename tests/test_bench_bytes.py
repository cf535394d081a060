"""The benchmark's algorithmic byte count for one verify pass, written out
independently at the 8B shape (d 4096, 36 layers, 32/8 heads of 128,
d_ff 12288, vocab 151936, bf16) with B = 1, gamma = 4 and 256 keys read."""
import bench
from synth import SHAPES


def test_verify_pass_bytes_8b():
    per_layer = (32 + 2 * 8) * 128 * 4096 + 4096 * 4096 + 2 * 12288 * 4096 + 4096 * 12288
    weights = (36 * per_layer + 151936 * 4096) * 2          # every linear weight once, bf16
    assert weights == 15_136_194_560
    kv_tok = 36 * 8 * 128 * 2 * 2                          # K and V rows of one position, all layers
    assert kv_tok == 147_456
    expect = (weights
              + 5 * 4096 * 2                               # the 5 gathered embedding rows
              + (2 * 36 + 1) * 4096 * 4                    # norm gains
              + 256 * kv_tok + 5 * kv_tok                  # KV read and written
              + 2 * 5 * 151936 * 4)                        # logits written and read once
    assert bench.verify_pass_bytes(SHAPES["qwen3_8b"], 1, 5, 256) == expect
    assert abs(expect / 1e9 - 15.18) < 0.005
