"""Early-exit verification (rows swept in position order, skipped after a
sequence's first rejection) against the full sweep and the oracle.

[R] "Speculative Decoding", 3. Accept or Reject: stop at the first rejection
and discard every later draft token -- so the rows after it cannot change the
result, and the early-exit path must give spec_verify_sample's outputs bit for
bit.
"""
import numpy as np
import pytest
import torch

import lossless_draft_verification_03_amd as _binding
import oracle
from gen import make_workload
from parity import classify_sample, to_dev
import sentinel

L = sentinel.wrap(_binding)   # every output buffer sentinel-filled before each call

pytestmark = pytest.mark.gpu


def _both(w, T=None, ks=(0, -1, 1, 2, 3)):
    """The full sweep and early exit with each block size in ks (0 =
    automatic); asserts the early-exit outputs agree across block sizes."""
    t, d = to_dev(w["target"]), to_dev(w["draft"])
    x, u = to_dev(w["draft_tokens"]), to_dev(w["uniforms"])
    T = float(w["temperature"]) if T is None else T
    g = w["draft_tokens"].shape[1]
    a1, o1 = L.verify_sample(t, d, x, u, T)
    res = []
    for k in ks:
        if k > g + 1:
            continue
        a2, o2 = L.verify_sample(t, d, x, u, T, early_exit=True, positions_per_launch=k)
        res.append((a2.cpu().numpy(), o2.cpu().numpy()))
    for a, o in res[1:]:
        assert np.array_equal(a, res[0][0]) and np.array_equal(o, res[0][1])
    return (a1.cpu().numpy(), o1.cpu().numpy()), res[0]


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("tiny", dict(B=7, gamma=6, V=333, dtype="bf16", seed=3)),
    ("zipf32k", {}),
    ("b64g7v128k", {}),
    ("b64g7v128k", dict(draft_noise=3.0, B=32, seed=5)),   # low acceptance
    ("b64g7v128k", dict(draft_tokens="argmax", B=32, seed=6)),  # long accepted runs
])
def test_early_exit_equals_full_sweep(name, kw):
    w = make_workload(name, cache=not kw, **kw)
    (a1, o1), (a2, o2) = _both(w)
    assert np.array_equal(a1, a2)
    assert np.array_equal(o1, o2)


def test_early_exit_matches_oracle_on_zipf():
    w = make_workload("zipf32k", B=64, seed=11)
    _, (acc, out) = _both(w)
    oacc, oout, infos = oracle.verify_sample(w["target"], w["draft"], "f32", w["draft_tokens"], w["uniforms"],
                                             float(w["temperature"]))
    res = classify_sample(acc, out, oacc, oout, infos)
    assert not res["unexplained"], res["unexplained"]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,g,V", [(1, 1, 1), (3, 2, 3), (2, 3, 5), (5, 1, 4097), (2, 63, 300), (4, 5, 16385)])
def test_early_exit_edge_shapes(dt, B, g, V):
    w = make_workload("tiny", B=B, gamma=g, V=V, dtype=dt, seed=B * 100 + g)
    (a1, o1), (a2, o2) = _both(w, ks=(0, -1, 1, 2, 5, g, g + 1))
    assert np.array_equal(a1, a2) and np.array_equal(o1, o2)


def test_early_exit_block_size_checked():
    w = make_workload("tiny", B=2, gamma=4, V=100, seed=1)
    args = (to_dev(w["target"]), to_dev(w["draft"]), to_dev(w["draft_tokens"]), to_dev(w["uniforms"]), 1.0)
    for k in (-2, 6):
        with pytest.raises(L.SpecError):
            L.verify_sample(*args, early_exit=True, positions_per_launch=k)


def test_early_exit_all_accepted_and_invalid_tokens():
    w = make_workload("tiny", B=6, gamma=5, V=500, dtype="bf16", seed=9)
    w["draft"] = w["target"][:, :5].copy()           # q = p: every draft accepted
    (a1, o1), (a2, o2) = _both(w)
    assert np.all(a2 == 5) and np.array_equal(o1, o2) and np.array_equal(a1, a2)
    w = make_workload("tiny", B=6, gamma=5, V=500, dtype="bf16", seed=10)
    w["draft_tokens"][1, 0] = -1                      # invalid at the first position
    w["draft_tokens"][2, 4] = 500                     # invalid at the last position
    (a1, o1), (a2, o2) = _both(w)
    assert a2[1] == -1 and a2[2] == -1
    assert np.array_equal(a1, a2) and np.array_equal(o1, o2)
