"""Pins of the CPU oracle against what the pages and mathematics fix.

Every check here compares the oracle with something other than itself: a
closed form, exact rational arithmetic, exhaustive enumeration, a library
routine, or a special case whose answer is known by construction.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _logits_of(p):
    """Logits whose softmax (T = 1) is p (exact up to float64 rounding)."""
    p = np.asarray(p, np.float64)
    with np.errstate(divide="ignore"):
        return np.log(p)


# ----------------------------------------------------------------- decode
def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x4049, 0xFF80, 0x7F7F], np.uint16)
    got = oracle.decode(bits, "bf16")
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 0.0
    assert got[3] == 0.0 and math.copysign(1.0, got[3]) == -1.0
    assert got[4] == 3.140625              # 0x4049 = 1.5703125 * 2
    assert got[5] == -math.inf
    assert got[6] == (2.0 - 2.0 ** -7) * 2.0 ** 127   # largest finite bf16


# ---------------------------------------------------------------- softmax
def test_softmax_closed_forms():
    rng = np.random.default_rng(0)
    z = rng.normal(0, 3, 257)
    for T in (0.3, 0.7, 1.0, 2.5):
        p = oracle.softmax(z, T)
        assert abs(p.sum() - 1.0) < 1e-14
        i, j = 3, 100
        assert math.isclose(p[i] / p[j], math.exp((z[i] - z[j]) / T), rel_tol=1e-12)
        # shift invariance and temperature as a logit scale
        assert np.allclose(oracle.softmax(z + 17.25, T), p, rtol=1e-12, atol=0)
        assert np.allclose(oracle.softmax(z / T, 1.0), p, rtol=1e-12, atol=0)
    assert np.allclose(oracle.softmax(np.zeros(7), 0.9), np.full(7, 1 / 7), rtol=1e-15)
    # -inf logits carry zero probability
    p = oracle.softmax(np.array([0.0, -np.inf, np.log(3.0)]), 1.0)
    assert p[1] == 0.0 and math.isclose(p[2] / p[0], 3.0, rel_tol=1e-15)


def test_accept_ratio_cases():
    assert oracle.accept_ratio(0.2, 0.4) == 0.5
    assert oracle.accept_ratio(0.4, 0.2) == 2.0
    assert oracle.accept_ratio(0.1, 0.0) == math.inf
    assert oracle.accept_ratio(0.0, 0.0) == 0.0
    # min(1, p/q) * q == min(p, q)  (A(x) on the review page)
    rng = np.random.default_rng(1)
    for _ in range(100):
        p, q = rng.random(2)
        assert math.isclose(min(1.0, oracle.accept_ratio(p, q)) * q, min(p, q), rel_tol=1e-15)


# ----------------------------------------------------------- inverse CDF
def _exact_draw(w, u):
    ws = [Fraction(float(x)) for x in w]
    thr = Fraction(float(u)) * sum(ws)
    c = Fraction(0)
    for v, x in enumerate(ws):
        c += x
        if c > thr:
            return v
    raise AssertionError


def test_inverse_cdf_matches_exact_rationals_and_searchsorted():
    rng = np.random.default_rng(2)
    for trial in range(300):
        V = int(rng.integers(1, 40))
        w = rng.random(V) * (rng.random(V) < 0.7)
        if not w.sum() > 0:
            w[int(rng.integers(0, V))] = 0.5
        u = float(np.float32(rng.random()))
        y, info = oracle.inverse_cdf(w, u)
        assert y == _exact_draw(w, u)
        assert w[y] > 0.0
        c = np.cumsum(w)
        assert y == int(np.searchsorted(c, u * c[-1], side="right"))
        assert info["margin"] >= 0.0


def test_inverse_cdf_edges():
    w = np.array([0.0, 0.0, 1.0, 0.0, 3.0, 0.0])
    assert oracle.inverse_cdf(w, 0.0)[0] == 2          # u = 0 -> first positive mass
    assert oracle.inverse_cdf(w, 0.2499)[0] == 2
    assert oracle.inverse_cdf(w, 0.25)[0] == 4         # strict '>' at the edge
    assert oracle.inverse_cdf(w, np.nextafter(1.0, 0.0))[0] == 4
    with pytest.raises(ValueError):
        oracle.inverse_cdf(np.zeros(4), 0.5)


def test_argmax_first_is_lowest_index():
    z = np.array([1.0, 5.0, 2.0, 5.0, 5.0])
    assert oracle.argmax_first(z) == 1 == int(np.argmax(z))
    rng = np.random.default_rng(3)
    for _ in range(200):
        z = rng.integers(-3, 3, size=int(rng.integers(1, 50))).astype(np.float64)
        assert oracle.argmax_first(z) == int(np.argmax(z))


# --------------------------------------------- lossless identity (exact)
def _pieces_run(P, Q, x, j, draw_v):
    """Run the oracle with uniforms at the midpoints of one piece of the
    piecewise-constant map u -> output: accept at positions < j, reject at j
    (j < gamma), and the final draw in token draw_v's CDF interval."""
    g = len(x)
    u = np.empty(g + 1)
    for i in range(min(j, g)):
        r = min(1.0, P[i][x[i]] / Q[i][x[i]])
        u[i] = r / 2
    if j < g:
        r = min(1.0, P[j][x[j]] / Q[j][x[j]])
        u[j] = (r + 1.0) / 2
        w = np.maximum(0.0, P[j] - Q[j])
    else:
        w = P[g]
    for i in range(j + 1, g):
        u[i] = 0.5          # never consumed
    F = np.cumsum(w) / w.sum()
    lo = F[draw_v - 1] if draw_v > 0 else 0.0
    u[g] = (lo + F[draw_v]) / 2
    zt = np.array([_logits_of(P[i]) for i in range(g + 1)])
    zd = np.array([_logits_of(Q[i]) for i in range(g)])
    return oracle.verify_sample_seq(zt, zd, x, u, 1.0), w


@pytest.mark.parametrize("V,g", [(3, 1), (3, 3), (4, 2), (5, 2), (6, 2), (4, 3)])
def test_lossless_by_exact_enumeration(V, g):
    """Exact enumeration over draft tuples x ~ prod q_i and over the pieces of
    u.  Pins, per position k reached: P(out_k = y) = p_k(y) (the review
    page's claim that accepted plus residual mass recovers p), P(propose and
    accept a) = min(p_k, q_k)(a), and sum max(0, p-q) = 1 - sum min(p, q)."""
    rng = np.random.default_rng(100 * V + g)
    P = [rng.dirichlet(np.ones(V)) * 0.99 + 0.01 / V for _ in range(g + 1)]
    Q = [rng.dirichlet(np.ones(V)) * 0.99 + 0.01 / V for _ in range(g)]
    P = [p / p.sum() for p in P]
    Q = [q / q.sum() for q in Q]
    out_mass = [np.zeros(V) for _ in range(g + 1)]     # P(out_k = y, reach k)
    reach = np.zeros(g + 1)
    acc_mass = [np.zeros(V) for _ in range(g)]          # P(propose+accept a, reach k)
    for x in np.ndindex(*([V] * g)):
        x = np.array(x, np.int32)
        wx = float(np.prod([Q[i][x[i]] for i in range(g)]))
        for j in range(g + 1):
            m_acc = 1.0
            for i in range(j):
                m_acc *= min(1.0, P[i][x[i]] / Q[i][x[i]])
            if j < g:
                r = min(1.0, P[j][x[j]] / Q[j][x[j]])
                m_j = m_acc * (1.0 - r)
            else:
                m_j = m_acc
            if m_j == 0.0:
                continue
            w = np.maximum(0.0, P[j] - Q[j]) if j < g else P[g]
            for v in range(V):
                if w[v] == 0.0:
                    continue
                mass = wx * m_j * w[v] / w.sum()
                (jj, toks, _), _ = _pieces_run(P, Q, x, j, v)
                assert jj == j and toks == [int(t) for t in x[:j]] + [v]
                for k in range(j + 1):
                    reach[k] += mass
                    out_mass[k][toks[k]] += mass
                for k in range(j):
                    acc_mass[k][x[k]] += mass
    for k in range(g + 1):
        assert np.allclose(out_mass[k] / reach[k], P[k], atol=1e-12, rtol=0)
    for k in range(g):
        assert np.allclose(acc_mass[k] / reach[k], np.minimum(P[k], Q[k]), atol=1e-12, rtol=0)
        assert math.isclose(np.maximum(0, P[k] - Q[k]).sum(), 1 - np.minimum(P[k], Q[k]).sum(),
                            abs_tol=1e-15)


# ------------------------------------------------------ special cases
def test_q_equals_p_accepts_everything():
    rng = np.random.default_rng(4)
    V, g = 50, 5
    for _ in range(20):
        zt = rng.normal(0, 2, (g + 1, V))
        zd = zt[:g].copy()
        x = rng.integers(0, V, g)
        u = rng.random(g + 1)
        j, toks, _ = oracle.verify_sample_seq(zt, zd, x, u, 0.8)
        assert j == g
        p = np.exp((zt[g] - zt[g].max()) / 0.8)
        c = np.cumsum(p)
        assert toks[-1] == int(np.searchsorted(c, u[g] * c[-1], side="right"))


def test_one_hot_target_sample_equals_greedy():
    rng = np.random.default_rng(5)
    V, g = 30, 6
    for _ in range(50):
        hot = rng.integers(0, V, g + 1)
        zt = np.full((g + 1, V), -np.inf)
        zt[np.arange(g + 1), hot] = rng.normal(0, 1, g + 1)
        zd = rng.normal(0, 1, (g, V))
        x = np.where(rng.random(g) < 0.6, hot[:g], rng.integers(0, V, g))
        u = rng.random(g + 1)
        j, toks, _ = oracle.verify_sample_seq(zt, zd, x, u, 1.3)
        jg, toksg = oracle.verify_greedy_seq(zt, x)
        assert (j, toks) == (jg, toksg)


def test_one_hot_draft_accepts_with_probability_p_and_residual_excludes_x():
    V = 6
    p = np.array([0.1, 0.25, 0.05, 0.3, 0.2, 0.1])
    x = 3
    zt = np.stack([_logits_of(p), _logits_of(p)])
    zd = np.full((1, V), -np.inf)
    zd[0, x] = 0.0
    # accept iff u < p(x)/1
    for u0, acc in ((0.29, True), (0.31, False)):
        j, toks, info = oracle.verify_sample_seq(zt, zd, [x], [u0, 0.5], 1.0)
        assert (j == 1) == acc
        if not acc:
            w = info["w"] / info["w"].sum()
            expect = p.copy()
            expect[x] = 0.0
            assert np.allclose(w, expect / expect.sum(), atol=1e-15)


# ------------------------------------------ expected committed length
def _golden_E():
    rows = []
    with open(__file__.replace("test_oracle_pins.py", "golden/expected_length_eagle_math.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                g, a, E, s, c = line.split()
                rows.append((int(g), float(a), float(E), float(s), float(c)))
    return rows


def test_printed_expected_length_matches_closed_form():
    for g, a, E, s, c in _golden_E():
        exact = (1 - a ** (g + 1)) / (1 - a)
        assert abs(exact - E) <= 0.005 + 1e-12
        assert abs(exact / (1 + g * c) - s) <= 0.005 + 1e-12


@pytest.mark.slow
@pytest.mark.parametrize("row", range(3))
def test_oracle_mean_committed_length_matches_page(row):
    """Constant per-token acceptance alpha = sum min(p, q) at every position:
    the oracle's mean committed length (accept_len + 1) must match the page's
    E and the accept_len histogram must be the truncated geometric law."""
    g, a, E_printed, _, _ = _golden_E()[row]
    # V = 2: sum(min(p, q)) = 1 - |p0 - q0| = a
    d = 1.0 - a
    p = np.array([0.5 + d / 2, 0.5 - d / 2])
    q = np.array([0.5 - d / 2, 0.5 + d / 2])
    assert math.isclose(np.minimum(p, q).sum(), a, rel_tol=1e-12)
    rng = np.random.default_rng(10 + row)
    n = 12000
    zt = np.stack([_logits_of(p)] * (g + 1))
    zd = np.stack([_logits_of(q)] * g)
    lens = np.empty(n, np.int64)
    for s in range(n):
        x = rng.choice(2, size=g, p=q)
        u = rng.random(g + 1)
        lens[s], _, _ = oracle.verify_sample_seq(zt, zd, x, u, 1.0)
    committed = lens + 1
    E = (1 - a ** (g + 1)) / (1 - a)
    sigma = committed.std() / math.sqrt(n)
    assert abs(committed.mean() - E) < 5 * sigma
    assert abs(committed.mean() - E_printed) < 5 * sigma + 0.005
    expect = np.array([a ** k * (1 - a) for k in range(g)] + [a ** g]) * n
    obs = np.bincount(lens, minlength=g + 1)
    chi2 = float(((obs - expect) ** 2 / expect).sum())
    from scipy.stats import chi2 as chi2dist
    assert chi2dist.sf(chi2, g) > 1e-4


# --------------------------------- greedy equals target-only greedy
def test_greedy_speculation_equals_target_greedy_decoding():
    """Multi-round greedy speculative decoding over a bigram toy LM must give
    exactly the target-only argmax decoding (review page, "Does Using a
    Small Model's Answer Reduce Quality?"), ties included."""
    rng = np.random.default_rng(6)
    V, g, n_tok = 64, 5, 1000
    A = np.round(rng.normal(0, 2, (V, V)) * 2) / 2           # coarse: many ties
    Bq = A + rng.normal(0, 1.0, (V, V))
    ref = [int(rng.integers(0, V))]
    while len(ref) < n_tok + 1:
        ref.append(int(np.argmax(A[ref[-1]])))
    out = [ref[0]]
    rounds = 0
    while len(out) < n_tok + 1:
        s = out[-1]
        x = []
        prev = s
        for _ in range(g):
            t = int(np.argmax(Bq[prev])) if rng.random() < 0.7 else int(rng.integers(0, V))
            x.append(t)
            prev = t
        rows = np.stack([A[s]] + [A[t] for t in x])
        j, toks = oracle.verify_greedy_seq(rows, np.array(x))
        out.extend(toks)
        rounds += 1
    assert out[: n_tok + 1] == ref
    assert rounds < n_tok                     # more than one token per round


@pytest.mark.slow
def test_stochastic_speculation_reproduces_target_sequence_law():
    """Speculative sampling over a bigram toy LM (V = 4) draws 3-token
    continuations with exactly the target's law prod p(y_t | y_{t-1})."""
    from scipy.stats import chisquare
    rng = np.random.default_rng(7)
    V, g, L, n = 4, 2, 3, 16000
    Pz = rng.normal(0, 1.0, (V, V))
    Qz = Pz + rng.normal(0, 1.2, (V, V))
    P = np.exp(Pz) / np.exp(Pz).sum(1, keepdims=True)
    Q = np.exp(Qz) / np.exp(Qz).sum(1, keepdims=True)
    s0 = 1
    counts = np.zeros(V ** L)
    for _ in range(n):
        out = [s0]
        while len(out) < L + 1:
            prev = out[-1]
            x = []
            for _ in range(g):
                t = int(rng.choice(V, p=Q[prev]))
                x.append(t)
                prev = t
            ctx = [out[-1]] + x
            zt = np.stack([Pz[c] for c in ctx])
            zd = np.stack([Qz[c] for c in ctx[:g]])
            _, toks, _ = oracle.verify_sample_seq(zt, zd, np.array(x), rng.random(g + 1), 1.0)
            out.extend(toks)
        y = out[1: L + 1]
        counts[y[0] * V * V + y[1] * V + y[2]] += 1
    expect = np.array([P[s0, a] * P[a, b] * P[b, c]
                       for a in range(V) for b in range(V) for c in range(V)]) * n
    assert chisquare(counts, expect).pvalue > 1e-4


# ----------------------------------------------------------------- tree
def _dfs_deepest(zt, tok, parent):
    """Independent brute force: depth-first search from the root through
    children that carry their parent's argmax (numpy's first-max argmax),
    visiting children in index order; keeps the first deepest node found in
    index order."""
    N = len(parent)
    a = [int(np.argmax(zt[n])) for n in range(N)]
    kids = {n: [] for n in range(N)}
    for n in range(1, N):
        kids[int(parent[n])].append(n)
    best = (0, 0)                 # (depth, -index)
    stack = [(0, 0)]
    while stack:
        n, d = stack.pop()
        if (d, -n) > best:
            best = (d, -n)
        for c in kids[n]:
            if int(tok[c]) == a[n]:
                stack.append((c, d + 1))
    return best[0], -best[1], a


def test_tree_matches_independent_dfs_on_small_random_trees():
    from gen.synth import tree_parents
    rng = np.random.default_rng(8)
    for trial in range(300):
        N = int(rng.integers(1, 14))
        V = int(rng.integers(2, 6))
        parent = tree_parents(N, "random", rng)
        zt = rng.integers(0, 3, (N, V)).astype(np.float64)       # ties
        a = np.argmax(zt, axis=1)
        tok = np.where(rng.random(N) < 0.75, a[np.maximum(parent, 0)], rng.integers(0, V, N))
        d, path, toks = oracle.verify_tree_seq(zt, tok, parent)
        d2, n2, a2 = _dfs_deepest(zt, tok, parent)
        assert d == d2
        end = path[-1] if path else 0
        assert end == n2 and toks[-1] == a2[n2]
        assert len(path) == d and toks[:-1] == [int(tok[m]) for m in path]


def test_chain_tree_equals_linear_greedy():
    from gen.synth import tree_parents
    rng = np.random.default_rng(9)
    for _ in range(100):
        g = int(rng.integers(1, 9))
        V = int(rng.integers(2, 8))
        zt = rng.integers(0, 4, (g + 1, V)).astype(np.float64)
        a = np.argmax(zt, axis=1)
        x = np.where(rng.random(g) < 0.7, a[:g], rng.integers(0, V, g))
        j, toks = oracle.verify_greedy_seq(zt, x)
        node_tok = np.concatenate([[int(rng.integers(0, V))], x])
        d, path, ttoks = oracle.verify_tree_seq(zt, node_tok, tree_parents(g + 1, "chain"))
        assert d == j and ttoks == toks and path == list(range(1, j + 1))


def test_tree_planted_binary_answer_and_invalid_parents():
    from gen.synth import tree_parents
    N, V = 15, 10
    par = tree_parents(N, "binary")
    zt = np.zeros((N, V))
    best = np.arange(N) % V
    zt[np.arange(N), best] = 1.0
    tok = (best[np.maximum(par, 0)] + 1) % V        # nothing matches ...
    for n in (2, 6, 13):                            # ... except root -> 2 -> 6 -> 13
        tok[n] = best[par[n]]
    tok[4] = best[par[4]]                            # a shallower match elsewhere
    d, path, toks = oracle.verify_tree_seq(zt, tok, par)
    assert (d, path) == (3, [2, 6, 13]) and toks == [int(tok[2]), int(tok[6]), int(tok[13]), int(best[13])]
    # two equally deep matches: the lower index wins
    tok[1] = best[0]
    tok[3] = best[1]
    tok[7] = best[3]
    d, path, _ = oracle.verify_tree_seq(zt, tok, par)
    assert (d, path) == (3, [1, 3, 7])
    bad = par.copy()
    bad[5] = 7
    assert oracle.verify_tree_seq(zt, tok, bad)[0] == -1
    bad = par.copy()
    bad[0] = 0
    assert oracle.verify_tree_seq(zt, tok, bad)[0] == -1


# ------------------------------------------------------------- LM head
def test_lmhead_one_hot_rows_and_integer_exactness():
    from gen.synth import f32_to_bf16_bits
    rng = np.random.default_rng(11)
    d, V = 64, 300
    W = f32_to_bf16_bits(rng.normal(0, 0.02, (d, V)).astype(np.float32))
    H = np.zeros((3, d), np.float32)
    H[0, 5] = 1.0
    H[1, 63] = 1.0
    H[2, 0] = -2.0
    Z = oracle.lmhead_logits(f32_to_bf16_bits(H), W, col_block=128)
    Wf = oracle.decode(W, "bf16")
    assert np.array_equal(Z[0], Wf[5]) and np.array_equal(Z[1], Wf[63]) and np.array_equal(Z[2], -2 * Wf[0])
    # small integers are exact in bf16: compare with int64 matmul
    Hi = rng.integers(-8, 9, (7, d))
    Wi = rng.integers(-8, 9, (d, V))
    Z = oracle.lmhead_logits(f32_to_bf16_bits(Hi.astype(np.float32)),
                             f32_to_bf16_bits(Wi.astype(np.float32)), col_block=100)
    assert np.array_equal(Z, (Hi @ Wi).astype(np.float64))


def test_batched_wrappers_agree_with_per_sequence():
    from gen import make_workload
    w = make_workload("tiny")
    acc, out, _ = oracle.verify_sample(w["target"], w["draft"], w["dtype"], w["draft_tokens"],
                                       w["uniforms"], w["temperature"])
    j, toks, _ = oracle.verify_sample_seq(w["target"][0].astype(np.float64), w["draft"][0].astype(np.float64),
                                          w["draft_tokens"][0], w["uniforms"][0], float(w["temperature"]))
    assert acc[0] == j and list(out[0, :j + 1]) == toks and np.all(out[0, j + 1:] == -1)


def test_invalid_draft_token_makes_sequence_invalid():
    """The reading for drafted tokens outside [0, V): the whole sequence is
    flagged (accept_len -1, every output -1), whichever position holds it and
    whether or not an earlier position would already have been rejected."""
    rng = np.random.default_rng(4)
    g, V = 4, 9
    zt = rng.normal(0, 1, (g + 1, V))
    zd = rng.normal(0, 1, (g, V))
    u = np.full(g + 1, 0.5)
    for pos in range(g):
        for bad in (-1, V, V + 100):
            x = rng.integers(0, V, g)
            x[pos] = bad
            j, toks, info = oracle.verify_sample_seq(zt, zd, x, u, 1.0)
            assert j == -1 and toks == [] and info["tests"] == []
    # batched: the flagged row is all -1, its neighbours are verified as usual
    B = 3
    T3 = np.stack([zt] * B).astype(np.float32)
    D3 = np.stack([zd] * B).astype(np.float32)
    X = rng.integers(0, V, (B, g)).astype(np.int32)
    X[1, 3] = V
    acc, out, _ = oracle.verify_sample(T3, D3, "f32", X, np.full((B, g + 1), 0.5, np.float32), 1.0)
    assert acc[1] == -1 and np.all(out[1] == -1)
    assert acc[0] >= 0 and acc[2] >= 0 and out[0, acc[0]] >= 0 and out[2, acc[2]] >= 0


def test_lmhead_verify_planted_answers():
    """oracle.lmhead_verify against outcomes fixed by construction (it pins
    the feature-row layout: row b*(g+1)+i target, row b*g+i draft, row
    b*(g+1)+g the bonus row).  W = identity (d = V = 64), so a feature row
    is its own logit row.

    * Target row (b, i) is 60 at a planted token a[b][i] and 0 elsewhere, the
      draft rows are 0 (q uniform): p(a) rounds to 1 in float64, so x_i is
      accepted iff x_i = a[b][i], the residual at a rejection is one-hot at
      a[b][j], and the bonus is a[b][g]: the output is greedy verification
      against the planted tokens (the review's "Does Using a Small Model's
      Answer Reduce Quality?": a point-mass target turns the test into the
      greedy rule).
    * Draft features equal to the target features (q = p): every draft is
      accepted and the bonus is a[b][g]."""
    from gen.synth import f32_to_bf16_bits
    rng = np.random.default_rng(12)
    B, g, d = 5, 4, 64
    V = d
    W = f32_to_bf16_bits(np.eye(d, dtype=np.float32))
    a = rng.integers(0, V, (B, g + 1))
    Ht = np.zeros((B * (g + 1), d), np.float32)
    for b in range(B):
        for i in range(g + 1):
            Ht[b * (g + 1) + i, a[b, i]] = 60.0
    # drafts that match the planted tokens for the first m[b] positions
    m = np.array([0, 2, 4, 1, 3])
    x = rng.integers(0, V, (B, g)).astype(np.int32)
    for b in range(B):
        x[b, :m[b]] = a[b, :m[b]]
        if m[b] < g:
            x[b, m[b]] = (a[b, m[b]] + 1 + rng.integers(0, V - 1)) % V      # != a
    u = rng.uniform(0.01, 0.99, (B, g + 1)).astype(np.float32)
    Hd0 = np.zeros((B * g, d), np.float32)
    acc, out, _, zt, zd = oracle.lmhead_verify(f32_to_bf16_bits(Ht), f32_to_bf16_bits(Hd0), W, x, u, 1.0)
    assert zt.shape == (B, g + 1, V) and zd.shape == (B, g, V) and np.all(zd == 0)
    for b in range(B):
        assert acc[b] == m[b]
        assert list(out[b, :m[b] + 1]) == list(a[b, :m[b]]) + [a[b, m[b]]]
        assert np.all(out[b, m[b] + 1:] == -1)
    # q = p: draft feature row b*g+i is target feature row b*(g+1)+i
    Hd = np.stack([Ht[b * (g + 1) + i] for b in range(B) for i in range(g)])
    acc, out, _, _, _ = oracle.lmhead_verify(f32_to_bf16_bits(Ht), f32_to_bf16_bits(Hd), W, x, u, 1.0)
    assert np.all(acc == g)
    for b in range(B):
        assert list(out[b]) == list(x[b]) + [a[b, g]]
