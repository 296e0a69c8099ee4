"""Seeded synthetic inputs for batched draft verification.

This package builds the input tensors that both the CPU oracle and the HIP
library consume.  It contains none of the verification arithmetic: no
softmax, no accept test, no residual, no argmax-based verification.  The
only "model-like" computation it performs is what a drafter would do before
verification starts (sampling draft tokens from the draft distribution, via
the Gumbel-max trick, and, for the EAGLE-style workload, pushing draft
features through the LM head with a plain NumPy matmul), because the
verification step takes those drafted tokens as given inputs.
"""
from .configs import CONFIGS, get_config  # noqa: F401
from .synth import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_linear,
    make_lmhead,
    make_tree,
    make_tree_sample,
    make_workload,
)
