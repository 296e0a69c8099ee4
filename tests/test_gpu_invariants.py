"""Whole-decoding invariants of the GPU path, checked against what the pages
fix rather than against the oracle.

* Greedy speculation (draft, verify with spec_verify_greedy, commit, repeat)
  over a bigram toy language model reproduces target-only greedy decoding
  bit for bit over 1000 tokens, ties included ([R] "Does Using a Small
  Model's Answer Reduce Quality?": with greedy decoding the output equals
  the target's own; "Interpreting 'No Quality Loss' Precisely").
* Speculative sampling (spec_verify_sample) over a V = 4 bigram model
  commits 3-token continuations with exactly the target's law
  prod p(y_t | y_(t-1)) ([W] "The guarantee": the output follows the
  target distribution; [R] "Does Using a Small Model's Answer Reduce
  Quality?").
"""
import numpy as np
import pytest
import torch

import lossless_draft_verification_03_amd as _binding
from gen.synth import f32_to_bf16_bits
from parity import to_dev
import sentinel

L = sentinel.wrap(_binding)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("dt,V,g,S", [("f32", 64, 5, 32), ("bf16", 5000, 7, 16)])
def test_greedy_speculation_equals_target_greedy_decoding(dt, V, g, S):
    """S sequences decode in lockstep rounds: each drafts g tokens (the
    draft model's argmax with probability 0.7, else a random token), the
    target scores the g + 1 positions (rows of the bigram table A), the GPU
    verifies greedily, the accepted prefix and the corrected or bonus token
    are committed.  Every sequence must equal argmax decoding of A from its
    start token.  A is rounded to multiples of 1/2, so rows hold ties and the
    lowest-index rule is exercised; the values are exact in bf16."""
    rng = np.random.default_rng(6 + V)
    n_tok = 1000
    A = (np.round(rng.normal(0, 2, (V, V)) * 2) / 2).astype(np.float32)
    Bq = A + rng.normal(0, 1.0, (V, V))
    A_dev = to_dev(f32_to_bf16_bits(A) if dt == "bf16" else A)
    assert dt != "bf16" or np.array_equal((f32_to_bf16_bits(A).astype(np.uint32) << 16).view(np.float32), A)
    starts = rng.integers(0, V, S)
    refs = []
    for s0 in starts:
        r = [int(s0)]
        while len(r) < n_tok + 1:
            r.append(int(np.argmax(A[r[-1]])))
        refs.append(r)
    seqs = [[int(s0)] for s0 in starts]
    rounds = 0
    while min(len(q) for q in seqs) < n_tok + 1:
        X = np.empty((S, g), np.int32)
        for b in range(S):
            prev = seqs[b][-1]
            for i in range(g):
                t = int(np.argmax(Bq[prev])) if rng.random() < 0.7 else int(rng.integers(0, V))
                X[b, i] = t
                prev = t
        ctx = np.concatenate([np.array([q[-1] for q in seqs])[:, None], X], 1)       # [S, g+1]
        target = A_dev[torch.from_numpy(ctx.astype(np.int64)).cuda()]                 # rows of A, [S, g+1, V]
        acc, out = L.verify_greedy(target, to_dev(X))
        acc, out = acc.cpu().numpy(), out.cpu().numpy()
        for b in range(S):
            j = int(acc[b])
            assert 0 <= j <= g and np.all(out[b, j + 1:] == -1)
            seqs[b].extend(int(t) for t in out[b, :j + 1])
        rounds += 1
    for b in range(S):
        assert seqs[b][: n_tok + 1] == refs[b], b
    assert rounds < n_tok                      # some rounds commit more than one token


def test_stochastic_speculation_reproduces_target_sequence_law():
    """V = 4, gamma = 2, 3 committed tokens after the start token, 2^18
    sequences at once.  Drafts are drawn on the host from the draft rows,
    verification runs on the GPU; the histogram of the 64 possible
    continuations must fit prod p(y_t | y_(t-1)) (chi-square), and so must the
    law of the first token alone."""
    from scipy.stats import chisquare
    rng = np.random.default_rng(7)
    V, g, Lc, n = 4, 2, 3, 1 << 18
    Pz = rng.normal(0, 1.0, (V, V)).astype(np.float32)
    Qz = (Pz + rng.normal(0, 1.2, (V, V))).astype(np.float32)
    # the laws of the float32 logits, computed in float64
    P = np.exp(Pz.astype(np.float64))
    P /= P.sum(1, keepdims=True)
    Q = np.exp(Qz.astype(np.float64))
    Q /= Q.sum(1, keepdims=True)
    Pd, Qd = to_dev(Pz), to_dev(Qz)
    s0 = 1
    seq = np.full((n, 1 + Lc + g + 1), -1, np.int64)
    seq[:, 0] = s0
    ln = np.ones(n, np.int64)
    ar = np.arange(n)
    while ln.min() < Lc + 1:
        last = seq[ar, ln - 1]
        X = np.empty((n, g), np.int64)
        prev = last
        cq = np.cumsum(Q, 1)
        for i in range(g):
            r = rng.random(n)
            X[:, i] = np.minimum((r[:, None] >= cq[prev]).sum(1), V - 1)
            prev = X[:, i]
        ctx = np.concatenate([last[:, None], X], 1)
        ctx_d = torch.from_numpy(ctx).cuda()
        zt = Pd[ctx_d]                           # [n, g+1, V]
        zd = Qd[ctx_d[:, :g]].contiguous()       # [n, g, V]
        U = to_dev(rng.random((n, g + 1), dtype=np.float32))
        acc, out = L.verify_sample(zt, zd, to_dev(X.astype(np.int32)), U, 1.0)
        acc, out = acc.cpu().numpy().astype(np.int64), out.cpu().numpy().astype(np.int64)
        assert np.all((acc >= 0) & (acc <= g))
        for k in range(g + 1):
            take = (k <= acc) & (ln < Lc + 1)
            seq[ar[take], ln[take]] = out[take, k]
            ln = ln + take
    y = seq[:, 1: Lc + 1]
    assert np.all((y >= 0) & (y < V))
    cells = y[:, 0] * V * V + y[:, 1] * V + y[:, 2]
    counts = np.bincount(cells, minlength=V ** Lc)
    expect = np.array([P[s0, a] * P[a, b] * P[b, c] for a in range(V) for b in range(V) for c in range(V)]) * n
    p_all = chisquare(counts, expect).pvalue
    p_first = chisquare(np.bincount(y[:, 0], minlength=V), P[s0] * n).pvalue
    print("chi-square p-values: sequences", p_all, "first token", p_first)
    assert p_all > 1e-4 and p_first > 1e-4
