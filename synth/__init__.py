"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This package draws random numbers and nothing else: model weights, prompts,
the uniforms the sampler consumes, and the order-2 Markov-chain prompts of the
copy-heavy workload.  It holds none of the method's arithmetic (no forward
pass, no softmax, no accept/reject rule), so that the oracle and the GPU path
can both consume it without sharing any code that computes a result.
"""

from .gen import (  # noqa: F401
    MASTER_SEED,
    Shape,
    SHAPES,
    substream_seed,
    make_weights,
    make_prompt,
    make_uniforms,
    make_markov_table,
    markov_prompt,
    round_uniforms,
)
