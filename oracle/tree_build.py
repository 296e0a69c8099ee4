"""EAGLE-2 dynamic draft tree: expansion, re-ranking, tree-attention mask --
TEST INFRASTRUCTURE ONLY.

Part of the CPU oracle (see the package docstring): float64 NumPy, no code
shared with the HIP library.

Sources: [M] "EAGLE math", section "EAGLE-2: dynamic draft trees" (the
drafter's own confidence stands in for the acceptance probability: grow the
tree greedily by expanding the nodes with the highest cumulative draft
probability, prune low-probability paths, re-rank which candidates to keep;
the number of nodes verified per target pass stays fixed; a tree attention
mask lets every candidate be scored in the one verification pass); [R]
"EAGLE-3 speculative decoding review", sections "EAGLE-2: Does Every Context
Need the Same Draft Tree?" (expand high-confidence branches, prune unlikely
ones; the mask lets a node see only the shared prefix and its own ancestors)
and "The Complete EAGLE-3 Inference Process" (2. Generate a Draft Tree).

Reading (the pages give the rule, not the procedure):

* A node's score is its cumulative draft log-probability: the sum of
  log q(token) along its root path, q = softmax(z_d / T) of the parent's
  draft row.  The root (the last committed token) scores 0.
* One expansion step: every node of the current frontier contributes the k
  tokens of its draft row with the highest q (equal logits: lower token
  index first) as children.  Children are appended to the node table, parent
  slot f of the frontier first, rank r within the row second (table position
  off + f*k + r).  The K children with the highest score (equal scores:
  lower table position) form the next frontier.
* Re-ranking: the root plus the M drafted nodes with the highest score
  (equal scores: shallower first, then lower table position) make the tree.
  A child never scores above its parent (log q <= 0) and wins a tie against
  it only if it were shallower, which it is not, so the kept set contains
  every kept node's parent.
* Output order: by depth, then score (higher first), then table position;
  parent[i] < i holds.  mask[i] has bit j set iff node j is node i or one of
  its ancestors (the tree attention mask: node i attends to the committed
  prefix and to exactly these tree nodes).

Node table, per sequence: parent (table index, -1 for the root and for
placeholders), token, score (float64, -inf for placeholders), depth.
"""
import numpy as np

NEG_INF = -np.inf


def log_softmax(z, T):
    """log q over the whole row, q = softmax(z / T); float64."""
    z = np.asarray(z, np.float64)
    a = (z - z.max()) / T
    return a - np.log(np.exp(a).sum())


def topk_tokens(z, k):
    """The k tokens with the largest logits, equal logits by lower index
    (the same order as by q, since q is increasing in z)."""
    z = np.asarray(z, np.float64)
    order = np.lexsort((np.arange(z.size), -z))
    return order[:k]


def expand_step(table, frontier, rows, T, k, K_out, off):
    """One depth of expansion for one sequence.

    table     dict of arrays parent, token, score, depth (modified in place)
    frontier  [K_in] table indices of the nodes to expand (-1 = empty slot)
    rows      [K_in, V] float64 draft logits of those nodes
    Returns the next frontier [K_out] (table indices, -1 padded)."""
    K_in = len(frontier)
    for f in range(K_in):
        for r in range(k):
            pos = off + f * k + r
            table["parent"][pos] = -1
            table["token"][pos] = -1
            table["score"][pos] = NEG_INF
            table["depth"][pos] = -1
        pn = int(frontier[f])
        if pn < 0:
            continue
        lq = log_softmax(rows[f], T)
        for r, tok in enumerate(topk_tokens(rows[f], k)):
            pos = off + f * k + r
            table["parent"][pos] = pn
            table["token"][pos] = int(tok)
            table["score"][pos] = table["score"][pn] + lq[tok]
            table["depth"][pos] = table["depth"][pn] + 1
    cand = [off + i for i in range(K_in * k) if table["score"][off + i] > NEG_INF]
    cand.sort(key=lambda p: (-table["score"][p], p))
    nxt = np.full(K_out, -1, np.int64)
    nxt[:min(K_out, len(cand))] = cand[:K_out]
    return nxt


def new_table(cap, root_token):
    t = {"parent": np.full(cap, -1, np.int64), "token": np.full(cap, -1, np.int64),
         "score": np.full(cap, NEG_INF), "depth": np.full(cap, -1, np.int64)}
    t["token"][0] = root_token
    t["score"][0] = 0.0
    t["depth"][0] = 0
    return t


def build_tree(table, n_nodes, M):
    """Re-rank the first n_nodes table entries and lay out the tree.

    Returns dict(n, parent, token, depth, table_index, mask) where mask is a
    [n, n] bool array (mask[i, j]: node i attends to node j)."""
    drafted = [p for p in range(1, n_nodes) if table["parent"][p] >= 0 and table["score"][p] > NEG_INF]
    drafted.sort(key=lambda p: (-table["score"][p], table["depth"][p], p))
    keep = [0] + drafted[:M]
    keep.sort(key=lambda p: (table["depth"][p], -table["score"][p], p))
    where = {p: i for i, p in enumerate(keep)}
    n = len(keep)
    parent = np.array([-1] + [where[int(table["parent"][p])] for p in keep[1:]], np.int64)
    mask = np.zeros((n, n), bool)
    for i in range(n):
        j = i
        while j >= 0:
            mask[i, j] = True
            j = int(parent[j])
    return {"n": n, "parent": parent, "token": np.array([table["token"][p] for p in keep], np.int64),
            "depth": np.array([table["depth"][p] for p in keep], np.int64),
            "table_index": np.array(keep, np.int64), "mask": mask}


def build_dynamic_tree(root_token, draft_rows_fn, T, k, K, depth, M):
    """The whole EAGLE-2 loop for one sequence: `depth` expansion steps, then
    re-ranking.  draft_rows_fn(table, frontier) returns the draft logits
    [len(frontier), V] of the frontier nodes (the drafter in the loop)."""
    cap = 1 + k + (depth - 1) * K * k
    table = new_table(cap, root_token)
    frontier = np.array([0])
    off = 1
    for d in range(depth):
        rows = draft_rows_fn(table, frontier)
        nxt = expand_step(table, frontier, rows, T, k, K, off)
        off += len(frontier) * k
        frontier = nxt
    return table, off, build_tree(table, off, M)
