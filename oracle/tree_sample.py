"""Stochastic (sampling) verification of a draft tree -- TEST INFRASTRUCTURE ONLY.

Part of the CPU oracle (see the package docstring): float64 NumPy, no code
shared with the HIP library.

Source: [R] "EAGLE-3 speculative decoding review", section "The Complete
EAGLE-3 Inference Process", step 4 (Strict Acceptance): for sampling, use
min(1, p/q) acceptance and residual correction to preserve the target
distribution -- on a tree.  [R] "Speculative Decoding" (3. Accept or Reject)
and "Does Using a Small Model's Answer Reduce Quality?" (A(x) = min(1,
p(x)/q(x)); resample from norm(max(0, p - q))) give the single-candidate
step this generalises.

Reading (the pages name the rule for trees but give no procedure for
siblings): the children of a node were drawn independently from the draft
distribution q of that node's draft row.  Starting at the root with p = the
node's target distribution, the children are tried in increasing node index;
child c with token x is accepted iff u[c] < p_i(x) / q(x), where p_1 = p and,
after each rejected sibling, p_{i+1} = norm(max(0, p_i - q)).  Each test is
one step of rejection sampling of p_i with proposal q, so the committed token
at every node has law p (multi-draft recursive rejection sampling).  An
accepted child becomes the current node.  If every child is rejected, one
token is drawn from the last residual p_{m+1}; at a node without children the
bonus token is drawn from p.  Uniforms: u[n] (n >= 1) is node n's test; u[0],
the root's slot (the root is never tested), is the final draw.  As for a
chain of drafts, a token outside [0, V) on any node but the root makes the
sequence invalid (accept_len = -1).

Second reading, for children drawn WITHOUT replacement (EAGLE-2 keeps k
distinct candidates per node, [M] "EAGLE-2: dynamic draft trees"; a sampling
drafter that wants k distinct children draws them one after another from q
with the earlier ones removed, as the Gumbel-top-k trick does in one go):
child k's proposal is q_k = q restricted to the tokens not yet drafted at the
node, renormalised, and every test and residual uses q_k in place of q:
accept iff u[c] < p_k(x) / q_k(x), then p_{k+1} = norm(max(0, p_k - q_k)).
Each test is again one rejection-sampling step of p_k with the proposal the
child was actually drawn from, so the committed token has law p.  A proposal
with no mass left gives q_k(x) = 0 (the ratio rule's +inf or 0).
"""
import numpy as np

from .verify import accept_ratio, inverse_cdf, residual, softmax, tree_is_valid


def children_of(parent):
    kids = [[] for _ in range(len(parent))]
    for c in range(1, len(parent)):
        kids[int(parent[c])].append(c)
    return kids


def verify_tree_sample_seq(zt, zd, node_tokens, parent, u, T, siblings="iid"):
    """One sequence.  zt, zd [N, V]: target and draft rows of every node (row
    n of zd is the draft distribution n's children were drawn from).
    siblings: "iid" (children drawn independently from q) or
    "without_replacement" (drawn one after another from q without
    replacement; see the module docstring).
    Returns (accept_len, path, tokens, info): accept_len = depth of the last
    accepted node (-1 for an invalid tree), path = accepted nodes from the
    root down (root excluded), tokens = their tokens then the final token.
    info: tests [(node, u, r)], draw (inverse_cdf info), w (the final draw's
    weights, unnormalised)."""
    zt = np.asarray(zt, np.float64)
    zd = np.asarray(zd, np.float64)
    V = zt.shape[1]
    if not tree_is_valid(parent) or any(not 0 <= int(t) < V for t in np.asarray(node_tokens)[1:]):
        return -1, [], [], dict(tests=[], draw=None, w=None)
    kids = children_of(parent)
    tests = []
    path = []
    n = 0
    while True:
        p = softmax(zt[n], T)
        if not kids[n]:
            w = p                                   # bonus at a leaf
            break
        q = softmax(zd[n], T)
        cur = p
        prop = q                                    # the law the next child was drawn from
        nxt = None
        for c in kids[n]:
            x = int(node_tokens[c])
            r = accept_ratio(cur[x], prop[x])
            tests.append((c, float(u[c]), r))
            if float(u[c]) < r:
                nxt = c
                break
            res = residual(cur, prop)
            total = np.sum(res)
            if total > 0.0:                         # > 0 in exact arithmetic after a rejection
                cur = res / total
            if siblings == "without_replacement":   # the next child cannot be x again
                prop = prop.copy()
                prop[x] = 0.0
                left = np.sum(prop)
                if left > 0.0:
                    prop = prop / left
            elif siblings != "iid":
                raise ValueError(siblings)
        if nxt is None:
            w = cur                                 # every child rejected
            break
        path.append(nxt)
        n = nxt
    y, draw = inverse_cdf(w, u[0])
    tokens = [int(node_tokens[m]) for m in path] + [y]
    return len(path), path, tokens, dict(tests=tests, draw=draw, w=w)


def verify_tree_sample(target, draft, dtype, node_tokens, parent, uniforms, T, siblings="iid"):
    """Batched: target, draft [B, N, V]; parent [N] or [B, N]; uniforms [B, N].
    Returns (accept_len [B], path [B, N] -1 padded, tokens [B, N] -1 padded,
    infos)."""
    from .verify import decode
    B, N, _ = target.shape
    acc = np.empty(B, np.int32)
    paths = np.full((B, N), -1, np.int32)
    toks = np.full((B, N), -1, np.int32)
    infos = []
    par = np.asarray(parent)
    for b in range(B):
        pb = par if par.ndim == 1 else par[b]
        d, path, tk, info = verify_tree_sample_seq(decode(target[b], dtype), decode(draft[b], dtype),
                                                   node_tokens[b], pb, uniforms[b], T, siblings)
        acc[b] = d
        paths[b, :len(path)] = path
        toks[b, :len(tk)] = tk
        infos.append(info)
    return acc, paths, toks, infos
