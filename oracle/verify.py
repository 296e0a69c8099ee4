"""Oracle functions (float64 NumPy).  Test infrastructure only.

Readings taken where the pages leave a step open (each is repeated at the
function that uses it):

* Temperature: p = softmax(z_target / T), q = softmax(z_draft / T), same T
  for both; the pages only say that temperature 0 means greedy.
* Uniforms: u[i] (i < gamma) is the accept test of drafted position i;
  u[gamma] is the one final draw (residual or bonus).
* Accept test: strict ``u < p(x)/q(x)`` with u in [0, 1), which accepts with
  probability exactly min(1, p/q).  q(x) = 0: ratio +inf if p(x) > 0, else 0.
* Final draw: inverse CDF in ascending vocabulary order, y = the first v
  with cumulative mass > u * total; if rounding leaves none, the last token
  with positive mass.  A zero residual after a rejection (impossible in
  exact arithmetic) falls back to p.
* Argmax ties: lowest index.
* Invalid drafts: a drafted token outside [0, V) at any position makes the
  sequence's verification invalid: accept_len = -1 and no tokens (the
  tree sampler applies the same rule to its nodes).
* Tree: parent[0] = -1 and 0 <= parent[i] < i; node 0 is the already
  committed token and is not verified; a node's token is checked against
  the argmax of its parent's row; among equally deep matching nodes the
  lowest index wins.
"""
import math

import numpy as np


# ------------------------------------------------------------------ inputs
def decode(arr, dtype):
    """Exact float64 values of logits stored as float32 or bf16 bit patterns.

    A bf16 value is the float32 whose upper 16 bits are the stored pattern
    and whose lower 16 bits are zero.
    """
    a = np.asarray(arr)
    if dtype == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    if dtype == "f64":
        return a.astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------- distributions
def softmax(z, T):
    """p = softmax(z / T) over the whole vocabulary.

    [R] "EAGLE: Predict Features, Not Tokens": the LM head output z goes
    through a softmax to give the next-token distribution; [M] "EAGLE's
    move" / "The uncertainty problem": p = softmax(LM_head(f')).  Temperature
    divides the logits (reading stated in the module docstring).  The max is
    subtracted before exponentiation; this changes nothing mathematically.
    """
    z = np.asarray(z, dtype=np.float64)
    T = float(T)
    m = np.max(z)
    e = np.exp((z - m) / T)
    return e / np.sum(e)


def accept_ratio(p_x, q_x):
    """p(x)/q(x), the quantity u is compared with.

    [R] "Does Using a Small Model's Answer Reduce Quality?", eq. for A(x):
    accept with probability min(1, p(x)/q(x)); [M] "Vanilla speculative
    decoding"; [W] "The mechanism".  q(x) = 0 can only come from underflow:
    the ratio is then +inf when p(x) > 0 (always accept) and 0 otherwise.
    """
    p_x = float(p_x)
    q_x = float(q_x)
    if q_x > 0.0:
        return p_x / q_x
    return math.inf if p_x > 0.0 else 0.0


def residual(p, q):
    """Unnormalised residual max(0, p - q).

    [R] "Does Using a Small Model's Answer Reduce Quality?", eq. for
    p_residual (norm of max(0, p - q)); [M] "(p - q)_+"; [W] "normalized
    residual max(0, p - q)".  Normalisation happens in the draw.
    """
    return np.maximum(0.0, np.asarray(p, np.float64) - np.asarray(q, np.float64))


def inverse_cdf(w, u):
    """Draw a token from the distribution proportional to w >= 0 using u in [0,1).

    Returns (y, info).  y is the first index whose cumulative mass exceeds
    u * total (ascending vocabulary order; a zero-mass token can never be
    the first to exceed it).  If rounding leaves no such index, y is the last
    index with positive mass.  ``info`` holds the normalised CDF ``F`` and
    the normalised threshold ``t`` so callers can measure decision margins.
    """
    w = np.asarray(w, np.float64)
    c = np.cumsum(w)
    total = c[-1]
    if not total > 0.0:
        raise ValueError("inverse_cdf: no positive mass")
    thr = float(u) * total
    above = np.flatnonzero(c > thr)
    if above.size:
        y = int(above[0])
    else:
        y = int(np.flatnonzero(w > 0.0)[-1])
    F = c / total
    t = thr / total
    lo = F[y - 1] if y > 0 else 0.0
    margin = min(t - lo, F[y] - t)
    return y, dict(F=F, t=t, margin=margin)


def argmax_first(z):
    """Index of the largest value; among equal maxima the lowest index.

    [R] "Does Using a Small Model's Answer Reduce Quality?": greedy
    decoding takes the target's argmax token.  Ties are broken toward the
    lowest index, the reading that keeps greedy output deterministic
    ([R] "Interpreting 'No Quality Loss' Precisely").
    """
    z = np.asarray(z)
    return int(np.flatnonzero(z == np.max(z))[0])


# ------------------------------------------------------------ per sequence
def verify_sample_seq(zt, zd, x, u, T):
    """Speculative sampling for one sequence.

    zt: target logits [gamma+1, V] (row i is the target distribution for
    drafted position i; row gamma is the bonus row).  zd: draft logits
    [gamma, V].  x: drafted tokens [gamma].  u: uniforms [gamma+1].

    Steps ([R] "Speculative Decoding", 3. Accept or Reject; [R] "Does Using
    a Small Model's Answer Reduce Quality?"; [M] "Vanilla speculative
    decoding"; [W] "The mechanism"):

    1. walk the drafted positions left to right; accept x_i with
       probability min(1, p_i(x_i)/q_i(x_i)), i.e. iff u[i] < p_i/q_i;
    2. at the first rejection j, discard every later draft and draw one
       token from norm(max(0, p_j - q_j)) with u[gamma];
    3. if every draft is accepted, draw the bonus token from p_gamma with
       u[gamma] ([M]: "+1 is the free bonus token").

    Returns (accept_len, tokens, info) with tokens = x_0..x_{j-1}, y.
    info["tests"] lists (i, u_i, r_i) for every accept test performed;
    info["draw"] is the inverse_cdf info of the final draw.

    A drafted token outside [0, V) (anywhere in x, the pages give no rule:
    reading stated in the module docstring) returns (-1, [], info) with no
    tests and no draw.
    """
    zt = np.asarray(zt, np.float64)
    zd = np.asarray(zd, np.float64)
    g = zd.shape[0]
    V = zt.shape[1]
    if any(not 0 <= int(t) < V for t in np.asarray(x)[:g]):
        return -1, [], dict(tests=[], draw=None, w=None)
    tests = []
    j = g
    for i in range(g):
        p = softmax(zt[i], T)
        q = softmax(zd[i], T)
        r = accept_ratio(p[x[i]], q[x[i]])
        tests.append((i, float(u[i]), r))
        if not (float(u[i]) < r):
            j = i
            break
    if j < g:
        p = softmax(zt[j], T)
        q = softmax(zd[j], T)
        w = residual(p, q)
        if not np.sum(w) > 0.0:
            w = p
    else:
        w = softmax(zt[g], T)
    y, draw = inverse_cdf(w, u[g])
    tokens = [int(t) for t in x[:j]] + [y]
    return j, tokens, dict(tests=tests, draw=draw, w=w)


def verify_greedy_seq(zt, x):
    """Greedy verification for one sequence.

    [R] "Does Using a Small Model's Answer Reduce Quality?": accept a draft
    iff it equals the target's argmax token; otherwise emit the target token
    and discard the rest.  If every draft matches, the bonus token is the
    argmax of row gamma ([R] "Speculative Decoding": take one more token
    already computed by the target).  The result equals target-only greedy
    decoding.
    """
    g = len(x)
    t = [argmax_first(zt[i]) for i in range(g + 1)]
    j = g
    for i in range(g):
        if int(x[i]) != t[i]:
            j = i
            break
    return j, [int(v) for v in x[:j]] + [t[j]]


def tree_is_valid(parent):
    parent = np.asarray(parent)
    if parent.size == 0 or parent[0] != -1:
        return False
    return all(0 <= int(parent[i]) < i for i in range(1, parent.size))


def verify_tree_seq(zt, node_tokens, parent):
    """Greedy tree verification for one sequence (brute force).

    [R] "EAGLE-2: Does Every Context Need the Same Draft Tree?" (a node sees
    only the shared prefix and its ancestors) and "The Complete EAGLE-3
    Inference Process", 4. Strict Acceptance: for greedy decoding accept the
    longest prefix matching the target's choices.  A root-to-node path is
    accepted iff every node on it, root excluded, carries the argmax of its
    parent's target row.  The deepest accepted node wins (lowest index among
    equals); the bonus token is the argmax of that node's own row.

    Returns (accept_len, path, tokens); accept_len = -1 for an invalid tree.
    """
    N = len(parent)
    if not tree_is_valid(parent):
        return -1, [], []
    a = [argmax_first(zt[n]) for n in range(N)]
    best_n, best_d = 0, 0
    for n in range(N):
        path = []
        m = n
        ok = True
        while m != 0:
            if int(node_tokens[m]) != a[int(parent[m])]:
                ok = False
                break
            path.append(m)
            m = int(parent[m])
        if ok and len(path) > best_d:
            best_n, best_d = n, len(path)
    path = []
    m = best_n
    while m != 0:
        path.append(m)
        m = int(parent[m])
    path.reverse()
    tokens = [int(node_tokens[m]) for m in path] + [a[best_n]]
    return best_d, path, tokens


# ----------------------------------------------------------------- batched
def verify_sample(target, draft, dtype, draft_tokens, uniforms, T):
    """verify_sample_seq over a batch; returns (accept_len[B], out[B,g+1], infos)."""
    B, g1, _ = target.shape
    acc = np.empty(B, np.int32)
    out = np.full((B, g1), -1, np.int32)
    infos = []
    for b in range(B):
        j, toks, info = verify_sample_seq(decode(target[b], dtype), decode(draft[b], dtype),
                                          draft_tokens[b], uniforms[b], T)
        acc[b] = j
        out[b, :len(toks)] = toks
        infos.append(info)
    return acc, out, infos


def verify_greedy(target, dtype, draft_tokens):
    B, g1, _ = target.shape
    acc = np.empty(B, np.int32)
    out = np.full((B, g1), -1, np.int32)
    for b in range(B):
        j, toks = verify_greedy_seq(decode(target[b], dtype), draft_tokens[b])
        acc[b] = j
        out[b, :len(toks)] = toks
    return acc, out


def verify_tree(target, dtype, node_tokens, parent):
    """parent is [N] (shared) or [B, N] (per sequence)."""
    B, N, _ = target.shape
    parent = np.asarray(parent)
    acc = np.empty(B, np.int32)
    path = np.full((B, N), -1, np.int32)
    out = np.full((B, N), -1, np.int32)
    for b in range(B):
        par = parent if parent.ndim == 1 else parent[b]
        d, p, toks = verify_tree_seq(decode(target[b], dtype), node_tokens[b], par)
        acc[b] = d
        path[b, :len(p)] = p
        out[b, :len(toks)] = toks
    return acc, path, out


# ----------------------------------------------------------------- LM head
def lmhead_logits(feat, W, col_block=8192):
    """z = W_LM h for every feature row, in float64.

    [R] "EAGLE: Predict Features, Not Tokens": the LM head turns the feature
    h_t into vocabulary logits z_t, and the draft reuses the target's LM
    head; [M] "EAGLE's move" / "Why feature drafting...": drafted features
    pass through the target's own, unchanged head.  No bias.  feat is bf16
    bits [M, d]; W is bf16 bits [d, V] (vocabulary innermost).  bf16
    products are exact in float64; columns are done in blocks so W is never
    widened whole.
    """
    H = decode(feat, "bf16")
    d, V = W.shape
    Z = np.empty((H.shape[0], V), np.float64)
    for c0 in range(0, V, col_block):
        c1 = min(V, c0 + col_block)
        Z[:, c0:c1] = H @ decode(W[:, c0:c1], "bf16")
    return Z


def lmhead_verify(feat_t, feat_d, W, draft_tokens, uniforms, T):
    """EAGLE-style verification: drafted features decoded through the
    target's own head, then verified like any draft.

    [R] "EAGLE: Predict Features, Not Tokens" (the draft reuses the target's
    LM head); [M] "EAGLE's move".  feat_t [B*(g+1), d]: row b*(g+1)+i is the
    target feature of position i of sequence b (i = g: the bonus row);
    feat_d [B*g, d]: row b*g+i is the drafted feature of position i; W bf16
    bits [d, V].  The logits of both go through verify_sample in float64.
    Returns (accept_len, out, infos, zt [B, g+1, V], zd [B, g, V])."""
    B, g = draft_tokens.shape
    zt = lmhead_logits(feat_t, W).reshape(B, g + 1, -1)
    zd = lmhead_logits(feat_d, W).reshape(B, g, -1)
    acc, out, infos = verify_sample(zt, zd, "f64", draft_tokens, uniforms, T)
    return acc, out, infos, zt, zd
