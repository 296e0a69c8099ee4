"""Pins of the KV-compaction oracle against what the pages state.

[R] "The Complete EAGLE-3 Inference Process", step 5: keep only the accepted
path's KV cache, drop rejected branches, resume drafting from the committed
prefix.  The central pin: after compaction the cache must hold exactly what
a plain left-to-right decode of the committed tokens would have cached.
"""
import numpy as np

import oracle
from oracle.kv import kv_compact, path_is_valid


def _entry(tokens, plane, E):
    """Synthetic KV entry of the last token of `tokens` seen in the context
    `tokens` (a stand-in for a layer's keys or values: a deterministic
    function of the context, different per plane)."""
    return np.random.default_rng([int(t) + 1 for t in tokens] + [1000 + plane]).integers(0, 256, E, dtype=np.uint8)


def _root_path(parent, n):
    p = []
    while n != 0:
        p.append(n)
        n = int(parent[n])
    return p[::-1]


def test_kv_compaction_resumes_from_committed_prefix():
    # A random tree is verified by the tree oracle; its nodes' entries were
    # computed in their own context (root path).  After compaction the cache
    # must equal the cache of a linear decode of the committed tokens.
    from gen.synth import tree_parents
    rng = np.random.default_rng(11)
    P, E, V = 3, 8, 12
    accepted_depths = set()
    for trial in range(40):
        N = int(rng.integers(2, 30))
        parent = tree_parents(N, "random", rng)
        zt = rng.normal(size=(N, V))
        a = zt.argmax(axis=1)
        # drafts: a node copies its parent's argmax with probability 0.7
        tok = np.where(rng.random(N) < 0.7, a[parent.clip(0)], rng.integers(0, V, N))
        tok[0] = rng.integers(0, V)
        d, path, _ = oracle.verify_tree_seq(zt, tok, parent)
        accepted_depths.add(d)
        L = int(rng.integers(0, 6))
        S = L + N + int(rng.integers(0, 3))
        prefix = rng.integers(0, V, L)
        cache = rng.integers(0, 256, (1, P, S, E), dtype=np.uint8)
        for n in range(N):
            ctx = list(prefix) + [tok[0]] + [tok[m] for m in _root_path(parent, n)]
            for p in range(P):
                cache[0, p, L + n] = _entry(ctx, p, E)
        out, new_len = kv_compact(cache, [L], [path], [d])
        assert new_len[0] == L + 1 + d
        committed = list(prefix) + [tok[0]] + [tok[m] for m in path]
        for t in range(d + 1):
            for p in range(P):
                assert np.array_equal(out[0, p, L + t], _entry(committed[:L + t + 1], p, E)), (trial, t, p)
        # the prefix is never touched
        assert np.array_equal(out[0, :, :L], cache[0, :, :L])
    assert len(accepted_depths) >= 3


def test_kv_linear_drafts_move_nothing():
    rng = np.random.default_rng(3)
    cache = rng.integers(0, 256, (4, 2, 20, 16), dtype=np.uint8)
    L = np.array([0, 3, 7, 10])
    d = np.array([0, 2, 5, 9])
    out, new_len = kv_compact(cache, L, None, d)
    assert np.array_equal(out, cache)
    assert list(new_len) == list(L + 1 + d)
    # the identity path given explicitly is the same as no path
    ident = np.array([[1 + i for i in range(9)]] * 4)
    out2, new_len2 = kv_compact(cache, L, ident, d)
    assert np.array_equal(out2, cache) and list(new_len2) == list(new_len)


def test_kv_chain_tree_verifies_to_the_identity_path():
    # a chain tree is a linear draft: the tree verifier's path is 1..d
    from gen.synth import tree_parents
    rng = np.random.default_rng(5)
    for _ in range(20):
        N = int(rng.integers(2, 12))
        parent = tree_parents(N, "chain")
        zt = rng.normal(size=(N, 9))
        a = zt.argmax(axis=1)
        tok = a[parent.clip(0)].copy()
        cut = int(rng.integers(1, N + 1))
        if cut < N:
            tok[cut] = (a[cut - 1] + 1) % 9
        d, path, _ = oracle.verify_tree_seq(zt, tok, parent)
        assert path == list(range(1, d + 1))
        cache = rng.integers(0, 256, (1, 2, N + 4, 8), dtype=np.uint8)
        out, new_len = kv_compact(cache, [2], [path], [d])
        assert np.array_equal(out, cache) and new_len[0] == 3 + d


def test_kv_overlapping_source_and_destination_slots():
    # path 2, 5, 6 after L = 3: slot 5 (= L + 2) is read for depth 1 and
    # written for depth 2; every read must see the cache before compaction
    S, E = 12, 4
    cache = np.zeros((1, 1, S, E), np.uint8)
    for s in range(S):
        cache[0, 0, s] = s
    out, new_len = kv_compact(cache, [3], [[2, 5, 6]], [3])
    assert new_len[0] == 7
    assert [int(out[0, 0, s, 0]) for s in range(S)] == [0, 1, 2, 3, 5, 8, 9, 7, 8, 9, 10, 11]


def test_kv_invalid_input_is_reported_and_left_alone():
    cache = np.arange(2 * 1 * 10 * 4, dtype=np.uint8).reshape(2, 1, 10, 4)
    cases = [
        ([2, 2], 2),        # not strictly increasing
        ([0, 1], 2),        # node 0 is the root, not a draft
        ([3, 8], 2),        # slot L + 8 = 10 is past the cache
    ]
    for path, d in cases:
        out, new_len = kv_compact(cache, [2, 2], [path, [1, 2]], [d, -1])
        assert list(new_len) == [-1, -1]
        assert np.array_equal(out, cache)
    assert path_is_valid([1, 4, 6], 2, 9) and not path_is_valid([1, 4, 7], 2, 9)
    assert not path_is_valid([1, 2, 3], 6, 9)           # L + 1 + d = 10 > S
