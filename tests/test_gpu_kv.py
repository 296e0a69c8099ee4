"""KV-cache compaction on the GPU against the CPU oracle (byte-exact).

[R] "The Complete EAGLE-3 Inference Process", 5. Update the KV Cache.
"""
import numpy as np
import pytest
import torch

import lossless_draft_verification_03_amd as _binding
import oracle
from gen import make_workload
from gen.synth import tree_parents
from oracle.kv import kv_compact as oracle_kv
from parity import to_dev
import sentinel

L = sentinel.wrap(_binding)   # every output buffer sentinel-filled before each call

pytestmark = pytest.mark.gpu


def _root_path(parent, n):
    p = []
    while n != 0:
        p.append(int(n))
        n = int(parent[n])
    return p[::-1]


def _paths(rng, B, N, S, invalid=True):
    """Per sequence: a random tree of N nodes, an accepted path (the root
    path of a random node), a prefix length that fits; some sequences get
    invalid input (rejected verify, non-increasing path, slots past S)."""
    path = np.full((B, N), -1, np.int32)
    acc = np.zeros(B, np.int32)
    pre = np.zeros(B, np.int32)
    for b in range(B):
        parent = tree_parents(N, "random", rng)
        p = _root_path(parent, int(rng.integers(0, N)))
        path[b, :len(p)] = p
        acc[b] = len(p)
        pre[b] = rng.integers(0, S - N + 1)
        if invalid and b % 7 == 3:
            kind = b % 3
            if kind == 0:
                acc[b] = -1
            elif kind == 1 and len(p) >= 2:
                path[b, 1] = path[b, 0]
            else:
                pre[b] = S - 1
    return pre, path, acc


@pytest.mark.parametrize("layout", ["seq_outer", "plane_outer"])
@pytest.mark.parametrize("E", [16, 48, 2048])
def test_kv_compact_matches_oracle(layout, E):
    rng = np.random.default_rng(E + (layout == "plane_outer"))
    B, P, N = 13, 5, 20
    S = N + 12
    cache = rng.integers(0, 256, (B, P, S, E), dtype=np.uint8)
    pre, path, acc = _paths(rng, B, N, S)
    want, want_len = oracle_kv(cache, pre, path, acc)
    if layout == "seq_outer":
        kv = to_dev(cache)
        view = kv
    else:
        kv = to_dev(np.ascontiguousarray(cache.transpose(1, 0, 2, 3)))
        view = kv.transpose(0, 1)
    new_len = L.kv_compact(view, to_dev(pre), to_dev(acc), to_dev(path))
    assert np.array_equal(new_len.cpu().numpy(), want_len)
    assert np.array_equal(view.cpu().numpy(), want)


def test_kv_compact_linear_drafts_touch_nothing():
    rng = np.random.default_rng(1)
    cache = rng.integers(0, 256, (6, 4, 16, 32), dtype=np.uint8)
    pre = np.array([0, 2, 5, 9, 14, 3], np.int32)
    acc = np.array([0, 3, 7, 6, 1, -1], np.int32)
    want, want_len = oracle_kv(cache, pre, None, acc)
    kv = to_dev(cache)
    new_len = L.kv_compact(kv, to_dev(pre), to_dev(acc))
    assert np.array_equal(new_len.cpu().numpy(), want_len)
    assert np.array_equal(kv.cpu().numpy(), cache)
    assert list(want_len) == [1, 6, 13, 16, 16, -1]


def test_kv_compact_after_gpu_tree_verify():
    # the tree verifier's outputs feed the compaction directly
    w = make_workload("tree63", B=6, V=1000)
    B, N = w["node_tokens"].shape
    acc, path, _ = L.verify_tree(to_dev(w["target"]), to_dev(w["node_tokens"]), to_dev(w["parent"]))
    oacc, opath, _ = oracle.verify_tree(w["target"], "bf16", w["node_tokens"], w["parent"])
    assert np.array_equal(acc.cpu().numpy(), oacc)
    rng = np.random.default_rng(7)
    S, P, E = N + 40, 3, 64
    cache = rng.integers(0, 256, (B, P, S, E), dtype=np.uint8)
    pre = rng.integers(0, S - N + 1, B).astype(np.int32)
    want, want_len = oracle_kv(cache, pre, opath, oacc)
    kv = to_dev(cache)
    new_len = L.kv_compact(kv, to_dev(pre), acc, path)
    assert np.array_equal(new_len.cpu().numpy(), want_len)
    assert np.array_equal(kv.cpu().numpy(), want)


def _pattern(b, P, S, E, dev=None):
    """Deterministic bytes of sequence b's planes (hash of the position)."""
    if dev is None:
        x = np.arange(P * S * E, dtype=np.int64) + b * P * S * E
        return (((x * 2654435761) & 0xFFFFFFFF) >> 24).astype(np.uint8).reshape(P, S, E)
    x = torch.arange(P * S * E, dtype=torch.int64, device=dev) + b * P * S * E
    return (((x * 2654435761) & 0xFFFFFFFF) >> 24).to(torch.uint8).view(P, S, E)


def test_kv_compact_full_size_sampled():
    # the benchmark's shape: 32 sequences, 64 planes (32 layers x K, V) of
    # 8 heads x 128 bf16 = 2048-byte entries, 63-node trees; offsets pass 2^31
    B, P, S, E, N = 32, 64, 576, 2048, 63
    rng = np.random.default_rng(3)
    pre, path, acc = _paths(rng, B, N, S, invalid=False)
    dev = torch.device("cuda")
    kv = torch.empty((B, P, S, E), dtype=torch.uint8, device=dev)
    for b in range(B):
        kv[b] = _pattern(b, P, S, E, dev)
    new_len = L.kv_compact(kv, to_dev(pre), to_dev(acc), to_dev(path))
    torch.cuda.synchronize()
    assert np.array_equal(new_len.cpu().numpy(), pre + 1 + acc)
    for b in (0, 1, 17, 31):
        want, _ = oracle_kv(_pattern(b, P, S, E)[None], pre[b:b + 1], path[b:b + 1], acc[b:b + 1])
        assert np.array_equal(kv[b].cpu().numpy(), want[0]), b
    del kv
    torch.cuda.empty_cache()
