"""Pins of the stochastic tree verification oracle.

[R] "The Complete EAGLE-3 Inference Process", 4. Strict Acceptance: for
sampling, min(1, p/q) acceptance and residual correction must preserve the
target distribution.  The central pin measures that exactly: over every
assignment of i.i.d. draft tokens to the tree's nodes and every piece of the
uniforms' space (explored through the oracle's own tests as a black box), the
first committed token must follow the root's target distribution, and the
next token the target distribution after it.
"""
import itertools

import numpy as np

import oracle
from oracle.tree_sample import children_of, verify_tree_sample_seq


def _law_over_uniforms(zt, zd, tok, parent, T, N, siblings="iid"):
    """Exact distribution of the committed tokens over the uniforms, found by
    exploring the oracle's accept tests depth first: each test splits the
    uniform's range at min(1, r); the final draw contributes its normalised
    weights.  Returns a list of (probability, first-token law or fixed
    tokens) items: (prob, tokens_prefix, draw_law)."""
    out = []
    stack = [({}, 1.0)]
    while stack:
        fixed, prob = stack.pop()
        u = np.full(N, 0.5)
        for c, v in fixed.items():
            u[c] = v
        d, path, tokens, info = verify_tree_sample_seq(zt, zd, tok, parent, u, T, siblings)
        undecided = [(c, r) for (c, _, r) in info["tests"] if c not in fixed]
        if not undecided:
            w = np.asarray(info["w"], np.float64)
            out.append((prob, tokens[:-1], w / w.sum()))
            continue
        c, r = undecided[0]
        pa = min(1.0, max(0.0, r))
        if pa > 0.0:
            stack.append(({**fixed, c: pa / 2}, prob * pa))
        if pa < 1.0:
            stack.append(({**fixed, c: (pa + 1.0) / 2}, prob * (1.0 - pa)))
    return out


def _path_model(V, seed):
    """Target and draft rows as functions of the token path (what a model's
    logits are), each row a fixed random distribution."""
    cache = {}

    def rows(path):
        key = tuple(path)
        if key not in cache:
            rng = np.random.default_rng([seed] + [t + 1 for t in key])
            zt = rng.normal(0, 1.2, V)
            zd = zt + rng.normal(0, 1.0, V)
            cache[key] = (zt, zd)
        return cache[key]
    return rows


def test_tree_sampling_preserves_the_target_distribution():
    # trees with sibling branching at the root and below; V = 3 tokens
    shapes = [
        [-1, 0, 0],                  # two siblings
        [-1, 0, 0, 0],               # three siblings
        [-1, 0, 0, 1, 2],            # two siblings, one child each
        [-1, 0, 1, 0, 1],            # mixed
    ]
    V, T = 3, 1.0
    for si, parent in enumerate(shapes):
        N = len(parent)
        model = _path_model(V, 40 + si)
        kids = children_of(parent)
        # every assignment of tokens to the non-root nodes; a node's children
        # are i.i.d. draws from the draft distribution after its path
        first = np.zeros(V)
        second = np.zeros((V, V))
        for assign in itertools.product(range(V), repeat=N - 1):
            tok = np.array([0] + list(assign))
            paths = [[]] * N
            for n in range(1, N):
                paths[n] = paths[parent[n]] + [int(tok[n])]
            weight = 1.0
            for n in range(N):
                q = oracle.softmax(model(paths[n])[1], T)
                for c in kids[n]:
                    weight *= q[tok[c]]
            zt = np.stack([model(paths[n])[0] for n in range(N)])
            zd = np.stack([model(paths[n])[1] for n in range(N)])
            for prob, prefix, law in _law_over_uniforms(zt, zd, tok, parent, T, N):
                pw = weight * prob
                if prefix:
                    first[prefix[0]] += pw
                    if len(prefix) >= 2:
                        second[prefix[0], prefix[1]] += pw
                    else:
                        second[prefix[0]] += pw * law
                else:
                    first += pw * law
        p_root = oracle.softmax(model([])[0], T)
        assert np.max(np.abs(first - p_root)) < 1e-12, (si, first, p_root)
        # given an accepted first token a, the next committed token follows
        # the target after a (only where a child can carry a)
        for a in range(V):
            if second[a].sum() > 1e-9:
                got = second[a] / second[a].sum()
                want = oracle.softmax(model([a])[0], T)
                assert np.max(np.abs(got - want)) < 1e-12, (si, a)


def _committed_law(shapes_and_models, V, T, siblings, distinct):
    """For each (parent, model): the exact law of the first committed token
    and of the second given the first, over the draft tokens (i.i.d. from q
    per node, or drawn without replacement: ordered distinct tuples, child k
    of a node weighted q(x_k) / (1 - sum of q over the earlier siblings))
    and over the uniforms."""
    out = []
    for parent, model in shapes_and_models:
        N = len(parent)
        kids = children_of(parent)
        first = np.zeros(V)
        second = np.zeros((V, V))
        for assign in itertools.product(range(V), repeat=N - 1):
            tok = np.array([0] + list(assign))
            if distinct and any(len({int(tok[c]) for c in kids[n]}) < len(kids[n]) for n in range(N)):
                continue
            paths = [[]] * N
            for n in range(1, N):
                paths[n] = paths[parent[n]] + [int(tok[n])]
            weight = 1.0
            for n in range(N):
                q = oracle.softmax(model(paths[n])[1], T)
                left = 1.0
                for c in kids[n]:
                    weight *= q[tok[c]] / left
                    if distinct:
                        left -= q[tok[c]]
            zt = np.stack([model(paths[n])[0] for n in range(N)])
            zd = np.stack([model(paths[n])[1] for n in range(N)])
            for prob, prefix, law in _law_over_uniforms(zt, zd, tok, parent, T, N, siblings):
                pw = weight * prob
                if prefix:
                    first[prefix[0]] += pw
                    if len(prefix) >= 2:
                        second[prefix[0], prefix[1]] += pw
                    else:
                        second[prefix[0]] += pw * law
                else:
                    first += pw * law
        out.append((first, second))
    return out


def _worst_error(laws, shapes_and_models, T):
    """Largest deviation of the committed laws from the target's."""
    err = 0.0
    for (first, second), (_, model) in zip(laws, shapes_and_models):
        err = max(err, np.max(np.abs(first - oracle.softmax(model([])[0], T))))
        for a in range(len(first)):
            if second[a].sum() > 1e-9:
                got = second[a] / second[a].sum()
                err = max(err, np.max(np.abs(got - oracle.softmax(model([a])[0], T))))
    return err


def test_without_replacement_siblings_preserve_the_target_distribution():
    # children drawn one after another without replacement (EAGLE-2's k
    # distinct candidates per node, sampled): exact enumeration over ordered
    # distinct sibling tuples.  V = 3 with three siblings makes the last
    # sibling's proposal a point mass on the one token left.
    cases = [
        ([-1, 0, 0], 4),
        ([-1, 0, 0, 0], 4),
        ([-1, 0, 0, 0], 3),
        ([-1, 0, 0, 1, 2], 4),
        ([-1, 0, 1, 0, 1, 1], 3),
    ]
    T = 0.8
    bias = []
    for ci, (parent, V) in enumerate(cases):
        sm = [(parent, _path_model(V, 70 + ci))]
        laws = _committed_law(sm, V, T, "without_replacement", distinct=True)
        assert _worst_error(laws, sm, T) < 1e-12, ci
        bias.append(_worst_error(_committed_law(sm, V, T, "iid", distinct=True), sm, T))
    # the i.i.d. rule applied to such children is biased (a residual that has
    # collapsed onto one token hides it, so not in every case): the pin tells
    # the two readings apart
    assert max(bias) > 1e-2, bias


def test_without_replacement_equals_iid_without_siblings():
    rng = np.random.default_rng(11)
    parent = np.array([-1, 0, 1, 2, 3])
    for trial in range(20):
        V = int(rng.integers(2, 30))
        zt = rng.normal(0, 2, (5, V))
        zd = zt + rng.normal(0, 1, (5, V))
        tok = rng.integers(0, V, 5)
        u = rng.random(5)
        a = verify_tree_sample_seq(zt, zd, tok, parent, u, 1.0, "iid")
        b = verify_tree_sample_seq(zt, zd, tok, parent, u, 1.0, "without_replacement")
        assert a[:3] == b[:3], trial


def test_without_replacement_rejects_a_repeated_sibling():
    # a token drafted twice at one node has no proposal mass the second time
    # and no residual target mass left after its first rejection
    rng = np.random.default_rng(5)
    parent = np.array([-1, 0, 0, 0])
    for trial in range(50):
        V = int(rng.integers(3, 12))
        zt = rng.normal(0, 2, (4, V))
        zd = rng.normal(0, 2, (4, V))
        x = int(rng.integers(0, V))
        y = (x + 1) % V
        tok = np.array([0, x, x, y])
        u = rng.random(4)
        u[1] = 0.999999                                  # the first x is rejected
        _, _, _, info = verify_tree_sample_seq(zt, zd, tok, parent, u, 1.0, "without_replacement")
        tests = {c: r for (c, _, r) in info["tests"]}
        if tests[1] < u[1]:
            assert tests[2] == 0.0, trial


def test_chain_tree_equals_linear_speculative_sampling():
    rng = np.random.default_rng(7)
    for trial in range(30):
        g, V, T = int(rng.integers(1, 6)), int(rng.integers(3, 40)), float(rng.choice([0.6, 1.0, 1.4]))
        zt = rng.normal(0, 2, (g + 1, V))
        zd = zt[:g] + rng.normal(0, 1, (g, V))
        x = np.array([int(np.argmax(zd[i] / T + rng.gumbel(size=V))) for i in range(g)])
        ul = rng.random(g + 1)
        acc, toks, _ = oracle.verify_sample_seq(zt, zd, x, ul, T)
        # the chain: node i+1 carries x_i; its test uses u_lin[i], the draw u_lin[g]
        parent = np.arange(-1, g)
        tok = np.concatenate([[0], x])
        ut = np.concatenate([[ul[g]], ul[:g]])
        zd_tree = np.concatenate([zd, np.zeros((1, V))])     # the leaf's draft row is never read
        d, path, ttoks, _ = verify_tree_sample_seq(zt, zd_tree, tok, parent, ut, T)
        assert d == acc and ttoks == toks and path == list(range(1, d + 1)), trial


def test_draft_equal_to_target_accepts_the_first_child_chain():
    rng = np.random.default_rng(3)
    parent = np.array([-1, 0, 0, 1, 1, 2, 3])
    N, V = len(parent), 20
    zt = rng.normal(0, 2, (N, V))
    tok = rng.integers(0, V, N)
    u = rng.random(N) * 0.999
    d, path, _, info = verify_tree_sample_seq(zt, zt.copy(), tok, parent, u, 1.0)
    assert path == [1, 3, 6] and d == 3                   # first child at every level
    assert all(r == 1.0 for (_, _, r) in info["tests"])


def test_invalid_tree():
    d, path, toks, _ = verify_tree_sample_seq(np.zeros((3, 4)), np.zeros((3, 4)), [0, 1, 2], [-1, 2, 0],
                                              [0.5] * 3, 1.0)
    assert d == -1 and path == [] and toks == []
    # an out-of-range token anywhere below the root, tested or not
    for bad in (-1, 4):
        d, path, toks, _ = verify_tree_sample_seq(np.zeros((3, 4)), np.zeros((3, 4)), [7, 1, bad], [-1, 0, 0],
                                                  [0.5] * 3, 1.0)
        assert d == -1 and path == [] and toks == []
    d, _, _, _ = verify_tree_sample_seq(np.zeros((3, 4)), np.zeros((3, 4)), [-5, 1, 3], [-1, 0, 0], [0.5] * 3, 1.0)
    assert d >= 0                                            # the root's token is never read
