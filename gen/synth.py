"""Seeded synthetic input builders.

Recipe (shared by every workload):

* One ``numpy.random.SeedSequence(seed)`` per workload, spawned into named
  child streams (target logits, draft noise, draft sampling, uniforms,
  extra).  Each sequence (or weight row block) draws from its own grandchild
  stream, so the values do not depend on the thread count.
* Normal draws are made in float32 and scaled in float64; logits are rounded
  to float32 and, for bf16 workloads, then to bf16 with round-to-nearest-even.
* Draft tokens are sampled from q = softmax(z_draft / T) of the *rounded*
  draft logits with the Gumbel-max trick (argmax of z/T + Gumbel noise),
  which draws exactly from that softmax without forming it.  This stands in
  for the drafter, which samples its proposals before verification begins.
* Uniforms are float32 in [0, 1).

bf16 tensors are returned as ``uint16`` bit patterns; float32 tensors as
``float32``.
"""
import hashlib
import json
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import get_config

_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + 0x7FFF + ((b >> 16) & 1)
    return (b >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _round(x64, dtype):
    x32 = np.asarray(x64, dtype=np.float32)
    return f32_to_bf16_bits(x32) if dtype == "bf16" else x32


def _as_f64(arr, dtype):
    return (bf16_bits_to_f32(arr) if dtype == "bf16" else arr).astype(np.float64)


# ------------------------------------------------------------ block drawing
def _parallel(n, fn):
    """Run fn(k) for k in range(n) on a thread pool (NumPy releases the GIL)."""
    if n == 1:
        fn(0)
        return
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fn, range(n)))


def _rng(seedseq):
    return np.random.Generator(np.random.PCG64(seedseq))


def _normal(rng, shape, std):
    return std * rng.standard_normal(shape, dtype=np.float32).astype(np.float64)


def _target_block(cfg, rng, nrows, V, ranks):
    z = _normal(rng, (nrows, V), cfg["target_std"])
    if cfg["logits"] == "zipf":
        # z = s*eps - a*ln(pi(v)), one permutation pi of 1..V for every row
        z -= cfg["zipf_slope"] * np.log(ranks)[None, :]
    elif cfg["logits"] != "normal":
        raise ValueError(cfg["logits"])
    return z


def _ranks(cfg, seedseq, V):
    if cfg["logits"] != "zipf":
        return None
    return _rng(seedseq).permutation(V).astype(np.float64) + 1.0


def _gumbel_max(rng, z64, T):
    """Index of max(z/T + Gumbel) per row: an exact draw from softmax(z/T)."""
    return np.argmax(z64 / T + rng.gumbel(size=z64.shape), axis=1).astype(np.int32)


# ------------------------------------------------------------- workloads
def make_linear(cfg):
    """Linear (chain) drafts: target [B,g+1,V], draft [B,g,V], tokens, uniforms.

    Each sequence b draws from its own child streams, so sequences can be
    generated in parallel and a larger B only appends sequences."""
    B, g, V, dt, T = cfg["B"], cfg["gamma"], cfg["V"], cfg["dtype"], float(cfg["temperature"])
    ss = np.random.SeedSequence(cfg["seed"]).spawn(5)
    ranks = _ranks(cfg, ss[4], V)
    kid_t, kid_n, kid_x = ss[0].spawn(B), ss[1].spawn(B), ss[2].spawn(B)
    odt = np.uint16 if dt == "bf16" else np.float32
    target = np.empty((B, g + 1, V), odt)
    draft = np.empty((B, g, V), odt)
    tokens = np.empty((B, g), np.int32)
    greedy_drafter = cfg.get("draft_tokens", "sample") == "argmax"

    def seq(b):
        target[b] = _round(_target_block(cfg, _rng(kid_t[b]), g + 1, V, ranks), dt)
        zd = _as_f64(target[b, :g], dt) + _normal(_rng(kid_n[b]), (g, V), cfg["draft_noise"])
        draft[b] = _round(zd, dt)
        zd = _as_f64(draft[b], dt)
        tokens[b] = (np.argmax(zd, axis=1) if greedy_drafter
                     else _gumbel_max(_rng(kid_x[b]), zd, T))

    _parallel(B, seq)
    uniforms = _rng(ss[3]).random((B, g + 1), dtype=np.float32)
    return dict(kind="linear", dtype=dt, B=B, gamma=g, V=V, temperature=np.float32(T),
                target=target, draft=draft, draft_tokens=tokens, uniforms=uniforms)


def tree_parents(N, shape="binary", rng=None):
    """Parent array with parent[0] = -1 and 0 <= parent[i] < i."""
    par = np.empty(N, np.int32)
    par[0] = -1
    for i in range(1, N):
        if shape == "binary":
            par[i] = (i - 1) // 2
        elif shape == "chain":
            par[i] = i - 1
        elif shape == "random":
            par[i] = rng.integers(0, i)
        elif shape == "star":
            par[i] = 0
        elif shape == "wide":
            # k = 4 children per node, breadth first
            par[i] = (i - 1) // 4
        else:
            raise ValueError(shape)
    return par


def make_tree(cfg):
    """Candidate tree: target [B,N,V], node_tokens [B,N], parent [N]."""
    B, N, V, dt = cfg["B"], cfg["N"], cfg["V"], cfg["dtype"]
    ss = np.random.SeedSequence(cfg["seed"]).spawn(5)
    parent = tree_parents(N, cfg.get("tree", "binary"), _rng(ss[4]))
    ranks = _ranks(cfg, ss[3], V)
    kid_t, kid_x = ss[0].spawn(B), ss[2].spawn(B)
    odt = np.uint16 if dt == "bf16" else np.float32
    target = np.empty((B, N, V), odt)
    node_tokens = np.empty((B, N), np.int32)

    def seq(b):
        target[b] = _round(_target_block(cfg, _rng(kid_t[b]), N, V, ranks), dt)
        # the drafter proposes its parent's target choice with probability p
        best = np.argmax(_as_f64(target[b], dt), axis=1)
        rng = _rng(kid_x[b])
        coin = rng.random(N) < cfg["match_prob"]
        rand_tok = rng.integers(0, V, size=N)
        tok = rand_tok.copy()
        tok[1:] = np.where(coin[1:], best[parent[1:]], rand_tok[1:])
        node_tokens[b] = tok

    _parallel(B, seq)
    return dict(kind="tree", dtype=dt, B=B, N=N, V=V, target=target,
                node_tokens=node_tokens, parent=parent)


def make_tree_sample(cfg):
    """Draft tree for sampling verification: target and draft rows [B,N,V]
    (row n belongs to node n), node tokens [B,N], parent [N] (or [B,N] for
    tree="random_per_seq"), uniforms [B,N].  The children of a node are
    independent Gumbel-max draws from q = softmax(draft row / T) of the
    parent, the way a sampling drafter grows the tree; with
    siblings="without_replacement", the m children of a node (in index order)
    are the m largest of one Gumbel-perturbed copy of the parent's draft row,
    best first: m draws from q one after another without replacement (the
    Gumbel-top-k trick), so a node needs m <= V."""
    B, N, V, dt, T = cfg["B"], cfg["N"], cfg["V"], cfg["dtype"], float(cfg["temperature"])
    ss = np.random.SeedSequence(cfg["seed"]).spawn(6)
    shape = cfg.get("tree", "binary")
    if shape == "random_per_seq":
        kid_p = ss[4].spawn(B)
        parent = np.stack([tree_parents(N, "random", _rng(kid_p[b])) for b in range(B)])
    else:
        parent = tree_parents(N, shape, _rng(ss[4]))
    ranks = _ranks(cfg, ss[5], V)
    kid_t, kid_n, kid_x = ss[0].spawn(B), ss[1].spawn(B), ss[2].spawn(B)
    odt = np.uint16 if dt == "bf16" else np.float32
    target = np.empty((B, N, V), odt)
    draft = np.empty((B, N, V), odt)
    node_tokens = np.zeros((B, N), np.int32)
    siblings = cfg.get("siblings", "iid")
    if siblings not in ("iid", "without_replacement"):
        raise ValueError(siblings)
    if siblings != "iid":
        for par in (parent if parent.ndim == 2 else parent[None]):
            if N > 1 and np.bincount(par[1:], minlength=N).max() > V:
                raise ValueError("a node has more children than there are tokens to draw without replacement")

    def seq(b):
        par = parent if parent.ndim == 1 else parent[b]
        target[b] = _round(_target_block(cfg, _rng(kid_t[b]), N, V, ranks), dt)
        zd = _as_f64(target[b], dt) + _normal(_rng(kid_n[b]), (N, V), cfg["draft_noise"])
        draft[b] = _round(zd, dt)
        if N > 1:
            zd = _as_f64(draft[b], dt)
            if siblings == "iid":
                node_tokens[b, 1:] = _gumbel_max(_rng(kid_x[b]), zd[par[1:]], T)
                return
            rng = _rng(kid_x[b])
            for n in range(N):
                kids = np.nonzero(par == n)[0]
                kids = kids[kids > 0]
                if len(kids) == 0:
                    continue
                g = zd[n] / T + rng.gumbel(size=V)
                m = len(kids)
                top = np.argpartition(-g, m - 1)[:m] if m < V else np.arange(V)
                node_tokens[b, kids] = top[np.argsort(-g[top], kind="stable")]

    _parallel(B, seq)
    uniforms = _rng(ss[3]).random((B, N), dtype=np.float32)
    return dict(kind="tree_sample", dtype=dt, B=B, N=N, V=V, temperature=np.float32(T), siblings=siblings,
                target=target, draft=draft, node_tokens=node_tokens, parent=parent, uniforms=uniforms)


def make_lmhead(cfg):
    """EAGLE-style inputs: features, LM head weight, draft tokens, uniforms."""
    B, g, d, V, T = cfg["B"], cfg["gamma"], cfg["d"], cfg["V"], float(cfg["temperature"])
    ss = np.random.SeedSequence(cfg["seed"]).spawn(6)
    Mt, Md = B * (g + 1), B * g
    ht = _round(_normal(_rng(ss[0]), (Mt, d), cfg["feat_std"]), "bf16")
    W = np.empty((d, V), np.uint16)
    blk = 64
    kid_w = ss[1].spawn((d + blk - 1) // blk)

    def wblock(k):
        r0, r1 = k * blk, min(d, (k + 1) * blk)
        W[r0:r1] = f32_to_bf16_bits(cfg["w_std"] * _rng(kid_w[k]).standard_normal((r1 - r0, V), dtype=np.float32))

    _parallel(len(kid_w), wblock)
    rows = (np.arange(B)[:, None] * (g + 1) + np.arange(g)[None, :]).reshape(-1)
    hd = _round(bf16_bits_to_f32(ht[rows]).astype(np.float64)
                + _normal(_rng(ss[2]), (Md, d), cfg["draft_noise"]), "bf16")
    # the drafter: its logits through the shared head (float32 BLAS), then a
    # Gumbel-max draw per drafted position
    zd = bf16_bits_to_f32(hd) @ bf16_bits_to_f32(W)
    tokens = _gumbel_max(_rng(ss[3]), zd.astype(np.float64), T)
    del zd
    uniforms = _rng(ss[4]).random((B, g + 1), dtype=np.float32)
    return dict(kind="lmhead", B=B, gamma=g, d=d, V=V, temperature=np.float32(T),
                feat_t=ht, feat_d=hd, W=W, draft_tokens=tokens.reshape(B, g),
                uniforms=uniforms)


_MAKERS = {"linear": make_linear, "tree": make_tree, "tree_sample": make_tree_sample, "lmhead": make_lmhead}
_CACHE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), ".cache", "specgen")


def make_workload(name, cache=False, **overrides):
    """Build (or load from the on-disk cache) the named workload."""
    cfg = get_config(name, **overrides)
    if not cache:
        return _MAKERS[cfg["kind"]](cfg)
    key = hashlib.sha1(json.dumps(cfg, sort_keys=True).encode()).hexdigest()[:16]
    path = os.path.join(_CACHE_DIR, f"{name}-{key}.npz")
    if os.path.exists(path):
        with np.load(path, allow_pickle=False) as f:
            out = {k: f[k] for k in f.files}
        for k in ("kind", "dtype", "siblings"):
            if k in out:
                out[k] = str(out[k])
        for k in ("B", "gamma", "V", "N", "d"):
            if k in out:
                out[k] = int(out[k])
        return out
    out = _MAKERS[cfg["kind"]](cfg)
    os.makedirs(_CACHE_DIR, exist_ok=True)
    tmp = path + f".tmp{os.getpid()}.npz"
    np.savez(tmp, **out)
    os.replace(tmp, path)
    return out
