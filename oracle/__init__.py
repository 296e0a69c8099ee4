"""CPU oracle for batched draft verification -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy statement of what the verification step
computes.  It exists to check the HIP library and nothing else: only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import
it.  The product path never calls it, and it shares no code, constants or
helpers with the library (the seeded input generators in ``gen`` feed both).

Sources (the three pages this method is described on):

* [R] "EAGLE-3 speculative decoding review" (6unoyunr.github.io blog)
* [M] "EAGLE math" (aicassindra.com, transformer_math series)
* [W] "Speculative decoding" (addictedtoai.net wiki)

Every function names the section it follows.  Every function here is pinned
by a CPU test against something other than itself (closed forms, exact
enumeration, exact rational arithmetic, special cases, brute force); none is
"parity unpinned".
"""
from .verify import (  # noqa: F401
    decode,
    softmax,
    accept_ratio,
    residual,
    inverse_cdf,
    argmax_first,
    verify_sample_seq,
    verify_greedy_seq,
    verify_tree_seq,
    verify_sample,
    verify_greedy,
    verify_tree,
    lmhead_logits,
    lmhead_verify,
)
from .kv import kv_compact  # noqa: F401
from .tree_build import build_dynamic_tree, build_tree, expand_step, new_table  # noqa: F401
from .tree_sample import verify_tree_sample, verify_tree_sample_seq  # noqa: F401
