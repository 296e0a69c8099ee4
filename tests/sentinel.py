"""The binding as the GPU tests use it: every output buffer is filled with a
sentinel before the call, so a kernel that skips a write cannot pass on
whatever memory the allocator hands back.

``wrap(L)`` returns a proxy of the binding module: the calls listed here get
freshly allocated outputs filled with SENT_I32 (int32), NaN (float) or 0xA5
(raw bytes) unless the test passes its own; everything else (constants,
workspaces, the raw library) is forwarded unchanged.  The sentinel is never
a valid output: token ids and lengths are >= -1, statistics are finite."""
import torch

SENT_I32 = -0x5A5A5A5A


def _i32(shape, dev):
    return torch.full(shape, SENT_I32, dtype=torch.int32, device=dev)


def _f(shape, dt, dev):
    return torch.full(shape, float("nan"), dtype=dt, device=dev)


class _Sentinel:
    def __init__(self, L):
        self._L = L

    def __getattr__(self, name):
        return getattr(self._L, name)

    def verify_sample(self, target, draft, draft_tokens, uniforms, temperature, out=None, **kw):
        B, g1, _ = target.shape
        if out is None:
            out = (_i32((B,), target.device), _i32((B, g1), target.device))
        return self._L.verify_sample(target, draft, draft_tokens, uniforms, temperature, out=out, **kw)

    def verify_greedy(self, target, draft_tokens, out=None, **kw):
        B, g1, _ = target.shape
        if out is None:
            out = (_i32((B,), target.device), _i32((B, g1), target.device))
        return self._L.verify_greedy(target, draft_tokens, out=out, **kw)

    def verify_tree(self, target, node_tokens, parent, out=None, **kw):
        B, N, _ = target.shape
        if out is None:
            out = (_i32((B,), target.device), _i32((B, N), target.device), _i32((B, N), target.device))
        return self._L.verify_tree(target, node_tokens, parent, out=out, **kw)

    def verify_tree_sample(self, target, draft, node_tokens, parent, uniforms, temperature, out=None, **kw):
        B, N, _ = target.shape
        if out is None:
            out = (_i32((B,), target.device), _i32((B, N), target.device), _i32((B, N), target.device))
        return self._L.verify_tree_sample(target, draft, node_tokens, parent, uniforms, temperature, out=out, **kw)

    def lmhead_project(self, feat, W, out=None, layout=None, **kw):
        layout = self._L.W_DV if layout is None else layout
        if out is None:
            M = feat.shape[0]
            V = W.shape[1] if layout == self._L.W_DV else W.shape[0]
            out = _f((M, V), torch.float32, feat.device)
        return self._L.lmhead_project(feat, W, out=out, layout=layout, **kw)

    def lmhead_verify(self, feat_t, feat_d, W, draft_tokens, uniforms, temperature, out=None, **kw):
        B, g = draft_tokens.shape
        if out is None:
            out = (_i32((B,), W.device), _i32((B, g + 1), W.device))
        return self._L.lmhead_verify(feat_t, feat_d, W, draft_tokens, uniforms, temperature, out=out, **kw)

    def row_stats(self, logits, temperature=1.0, want=3, ws=None, out=None):
        rows = logits.shape[0]
        if out is None:
            out = (_f((rows,), torch.float32, logits.device), _f((rows,), torch.float64, logits.device),
                   _i32((rows,), logits.device))
        return self._L.row_stats(logits, temperature, want, ws=ws, out=out)

    def row_partials(self, logits, temperature=1.0, want=1, out=None):
        if out is None:
            rows, V = logits.shape
            nseg = self._L.lib.spec_row_segments(V, self._L.dtype_code(logits))
            out = torch.full((rows, nseg, 24), 0xA5, dtype=torch.uint8, device=logits.device)
        return self._L.row_partials(logits, temperature, want, out=out)

    def probe_probs(self, target, draft, temperature, ws=None, out=None):
        if out is None:
            rows, V = target.shape
            out = tuple(_f((rows, V), torch.float64, target.device) if (k == 0 or draft is not None) else None
                        for k in range(3))
        return self._L.probe_probs(target, draft, temperature, ws=ws, out=out)

    def kv_compact(self, kv, prefix_len, accept_len, path=None, new_len=None):
        if new_len is None:
            new_len = _i32((kv.shape[0],), kv.device)
        return self._L.kv_compact(kv, prefix_len, accept_len, path, new_len=new_len)

    def tree_expand(self, draft_logits, frontier, table, off, temperature, k, K_out, ws=None, next_frontier=None):
        if next_frontier is None:
            next_frontier = _i32((draft_logits.shape[0], K_out), draft_logits.device)
        return self._L.tree_expand(draft_logits, frontier, table, off, temperature, k, K_out, ws=ws,
                                   next_frontier=next_frontier)

    def tree_build(self, table, n_nodes, M, out=None):
        if out is None:
            B = table[0].shape[0]
            dev = table[0].device
            W = (M + 1 + 31) // 32
            out = (_i32((B,), dev),) + tuple(_i32((B, M + 1), dev) for _ in range(4)) + (_i32((B, M + 1, W), dev),)
        return self._L.tree_build(table, n_nodes, M, out=out)


def wrap(L):
    return _Sentinel(L)
