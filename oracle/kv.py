"""KV-cache compaction to the accepted path -- TEST INFRASTRUCTURE ONLY.

Part of the CPU oracle (see the package docstring): plain NumPy, no code
shared with the HIP library.

Source: [R] "EAGLE-3 speculative decoding review", section "The Complete
EAGLE-3 Inference Process", step 5 (Update the KV Cache): only the cache of
the accepted path is kept, rejected branches are dropped, and drafting
resumes from the committed prefix; and section "Implementation Is More
Complex Than a Simple Two-Model Setup" (the serving system prunes the KV
cache to the accepted branch).

Reading (the pages fix no cache layout): sequence b had L_b tokens cached
before the verification forward.  That forward processed the tree's N nodes
-- node 0 is the root, the last committed token, and nodes 1..N-1 the
drafts -- and wrote node n's entry at slot L_b + n.  After verification the
committed sequence is the root followed by the accepted path
n_1 < n_2 < ... < n_d (node indices along a root path increase, since a
parent precedes its children), so its entries belong at slots L_b .. L_b + d:
slot L_b + t receives what node n_t's slot held before the compaction.  The
new cache length is L_b + 1 + d.  Every other slot keeps its contents.  A
linear draft is the chain n_t = t, for which nothing moves.

Invalid input (accept_len < 0, a path that is not strictly increasing from
1, or slots past the cache) leaves the sequence untouched and reports -1 as
its new length.
"""
import numpy as np


def path_is_valid(nodes, L, S):
    """1 <= n_1 < n_2 < ... and every slot used lies inside [0, S)."""
    prev = 0
    for n in nodes:
        if int(n) <= prev:
            return False
        prev = int(n)
    d = len(nodes)
    if L < 0 or L + 1 + d > S:
        return False
    return d == 0 or L + prev < S


def kv_compact(cache, prefix_len, path, accept_len):
    """Keep the accepted path's entries after the committed prefix.

    cache       [B, P, S, E] uint8: entry (b, plane p, slot s) = E bytes
                (a plane is one layer's keys or values).
    prefix_len  [B]: L_b.
    path        [B, >= d] node indices of the accepted path in depth order
                (the tree verifier's path output), or None for linear
                drafts (n_t = t).
    accept_len  [B]: d_b (-1 = the verifier rejected the input).
    Returns (new cache, new_len [B]); the input is not modified.
    """
    out = np.array(cache, copy=True)
    B, _, S, _ = cache.shape
    new_len = np.empty(B, np.int64)
    for b in range(B):
        d, L = int(accept_len[b]), int(prefix_len[b])
        if d < 0:
            new_len[b] = -1
            continue
        nodes = list(range(1, d + 1)) if path is None else [int(n) for n in path[b][:d]]
        if not path_is_valid(nodes, L, S):
            new_len[b] = -1
            continue
        before = np.array(cache[b], copy=True)       # every read sees the pre-compaction cache
        for t, n in enumerate(nodes, start=1):
            out[b, :, L + t] = before[:, L + n]
        new_len[b] = L + 1 + d
    return out, new_len
