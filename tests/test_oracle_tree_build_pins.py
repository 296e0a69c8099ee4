"""Pins of the EAGLE-2 tree-builder oracle against what the pages state.

[M] "EAGLE math", "EAGLE-2: dynamic draft trees": expand the nodes with the
highest cumulative draft probability, prune, re-rank; the node budget is
fixed; the mask lets every candidate be scored in one pass.  [R]
"EAGLE-2: Does Every Context Need the Same Draft Tree?": a node sees the
shared prefix and its own ancestors only.
"""
import itertools

import numpy as np

import oracle
from oracle.tree_build import build_dynamic_tree, build_tree, expand_step, log_softmax, new_table, topk_tokens


def _rows_fn(rng_seed, V, scale=2.0):
    """Synthetic drafter: a node's row is a fixed function of its table index."""
    def fn(table, frontier):
        out = np.zeros((len(frontier), V))
        for f, n in enumerate(frontier):
            out[f] = np.random.default_rng([rng_seed, int(n) + 1]).normal(0, scale, V)
        return out
    return fn


def _path_prob(table, p, rows_by_node, T):
    """Product of q along the root path, from softmax probabilities (an
    independent route to exp(score))."""
    prob = 1.0
    while table["parent"][p] >= 0:
        par = int(table["parent"][p])
        q = oracle.softmax(rows_by_node[par], T)
        prob *= q[int(table["token"][p])]
        p = par
    return prob


def _record_rows(fn):
    seen = {}

    def wrapped(table, frontier):
        rows = fn(table, frontier)
        for f, n in enumerate(frontier):
            if n >= 0:
                seen[int(n)] = rows[f]
        return rows
    return wrapped, seen


def test_topk_and_log_softmax_basics():
    z = np.array([1.0, 3.0, 3.0, -2.0, 3.0, 0.5])
    assert list(topk_tokens(z, 4)) == [1, 2, 4, 0]       # equal logits: lower index first
    lq = log_softmax(z, 0.7)
    assert abs(np.exp(lq).sum() - 1.0) < 1e-15
    assert np.allclose(np.exp(lq), oracle.softmax(z, 0.7), rtol=1e-14, atol=0)


def test_kept_nodes_are_the_most_probable_and_form_a_tree():
    rng = np.random.default_rng(0)
    for trial in range(12):
        V, T = int(rng.integers(6, 40)), float(rng.choice([0.5, 1.0, 1.7]))
        k, K, D, M = int(rng.integers(1, 5)), int(rng.integers(1, 5)), int(rng.integers(1, 5)), int(rng.integers(1, 20))
        fn, rows_by_node = _record_rows(_rows_fn(trial, V))
        table, n_nodes, tree = build_dynamic_tree(7, fn, T, k, K, D, M)
        drafted = [p for p in range(1, n_nodes) if table["parent"][p] >= 0]
        assert tree["n"] == 1 + min(M, len(drafted))                     # the budget
        probs = {p: _path_prob(table, p, rows_by_node, T) for p in drafted}
        for p in drafted:                                                 # score = log of the product
            assert abs(np.exp(table["score"][p]) - probs[p]) <= 1e-12 * max(1.0, probs[p]) + 1e-300
        kept = set(int(x) for x in tree["table_index"][1:])
        best = sorted(drafted, key=lambda p: -probs[p])[:M]
        if len(drafted) > M:
            gap = probs[best[-1]] - max(probs[p] for p in drafted if p not in best)
            if gap > 1e-12:
                assert kept == set(best), trial
        par = tree["parent"]
        assert par[0] == -1 and all(0 <= par[i] < i for i in range(1, tree["n"]))
        for i in range(1, tree["n"]):                                     # table parents are kept
            assert table["parent"][tree["table_index"][i]] == tree["table_index"][par[i]]
            assert tree["depth"][i] == tree["depth"][par[i]] + 1


def test_mask_is_the_ancestor_relation():
    rng = np.random.default_rng(1)
    fn = _rows_fn(5, 30)
    table, n_nodes, tree = build_dynamic_tree(3, fn, 1.0, 3, 4, 4, 25)

    def path(i):  # table indices from the root to kept node i
        out, p = [], int(tree["table_index"][i])
        while p >= 0:
            out.append(p)
            p = int(table["parent"][p])
        return tuple(out[::-1])
    paths = [path(i) for i in range(tree["n"])]
    for i in range(tree["n"]):
        for j in range(tree["n"]):
            # j is visible to i iff j's root path is a prefix of i's
            assert tree["mask"][i, j] == (paths[i][:len(paths[j])] == paths[j])


def test_one_depth_is_a_plain_top_m():
    rng = np.random.default_rng(2)
    z = rng.normal(0, 2, 50)
    T = 0.8
    table, n_nodes, tree = build_dynamic_tree(1, lambda t, f: z[None, :], T, 10, 10, 1, 6)
    q = oracle.softmax(z, T)
    assert list(tree["token"][1:]) == list(np.argsort(-q, kind="stable")[:6])
    assert list(tree["parent"]) == [-1] + [0] * 6


def test_one_child_one_frontier_is_greedy_drafting():
    V, D = 25, 6
    fn = _rows_fn(9, V)
    table, n_nodes, tree = build_dynamic_tree(4, fn, 1.0, 1, 1, D, D)
    # greedy drafting: each depth takes the argmax of the previous node's row
    node, toks = 0, []
    for d in range(D):
        row = fn(table, np.array([node]))[0]
        toks.append(int(np.argmax(row)))
        node = 1 + d
    assert list(tree["token"][1:]) == toks
    assert list(tree["parent"]) == [-1] + list(range(D))


def test_reranking_maximises_expected_accepted_length():
    # If the draft's confidence were the acceptance probability, a kept node
    # would be accepted with probability exp(score), so the expected number
    # of accepted tokens is the sum of exp(score) over kept nodes.  Re-ranking
    # must reach the maximum over every ancestor-closed set of M nodes.
    for seed in range(6):
        fn = _rows_fn(100 + seed, 8, scale=1.5)
        table, n_nodes, tree = build_dynamic_tree(0, fn, 1.0, 2, 2, 3, 4)
        drafted = [p for p in range(1, n_nodes) if table["parent"][p] >= 0]
        val = {p: np.exp(table["score"][p]) for p in drafted}
        best = 0.0
        for sub in itertools.combinations(drafted, 4):
            s = set(sub)
            if all(table["parent"][p] == 0 or table["parent"][p] in s for p in sub):
                best = max(best, sum(val[p] for p in sub))
        got = sum(val[int(p)] for p in tree["table_index"][1:])
        assert abs(got - best) < 1e-12, seed


def test_expand_step_frontier_and_placeholders():
    # hand-made step: two frontier nodes with known scores, one empty slot
    table = new_table(1 + 3 * 2, 0)
    table["parent"][1], table["token"][1], table["score"][1], table["depth"][1] = 0, 5, np.log(0.5), 1
    table["parent"][2], table["token"][2], table["score"][2], table["depth"][2] = 0, 6, np.log(0.25), 1
    rows = np.array([[0.0, np.log(3.0), -np.inf],     # q = (1/4, 3/4, 0)
                     [np.log(2.0), 0.0, -np.inf],     # q = (2/3, 1/3, 0)
                     [0.0, 0.0, 0.0]])
    table2 = {k: np.concatenate([v, np.full(6, v[-1])]) for k, v in table.items()}
    nxt = expand_step(table2, np.array([1, 2, -1]), rows, 1.0, 2, 3, 3)
    # children of node 1: tokens 1 (0.5*3/4), 0 (0.5/4); of node 2: tokens 0 (0.25*2/3), 1 (0.25/3)
    assert list(table2["token"][3:9]) == [1, 0, 0, 1, -1, -1]
    assert np.allclose(np.exp(table2["score"][3:7]), [0.375, 0.125, 1 / 6, 1 / 12], rtol=1e-14)
    assert list(table2["parent"][3:9]) == [1, 1, 2, 2, -1, -1]
    assert list(nxt) == [3, 5, 4]
