"""The verification calls (linear, early exit, greedy, trees and the
EAGLE-style LM head) under HIP graph capture and on concurrent streams.

The library allocates nothing, keeps no state between calls and enqueues
only kernels (and device-to-device copies) on the caller's stream, so a
serving loop can capture it into a graph or run independent batches on
separate streams with separate workspaces.  Each graph replay is checked
against the eager results, with eager work and synchronisations between the
replays, and once more after new inputs were copied into the captured
buffers.
"""
import numpy as np
import pytest
import torch

import lossless_draft_verification_03_amd as L
from gen import make_workload
from parity import to_dev

pytestmark = pytest.mark.gpu


class _Calls:
    """Fixed device buffers for one linear and one tree workload, the
    verification calls on them, and their outputs."""

    def __init__(self, seed):
        w = make_workload("b64g7v128k", B=8, V=20000, seed=seed)
        self.lin = {k: to_dev(w[k]) for k in ("target", "draft", "draft_tokens", "uniforms")}
        self.T = float(w["temperature"])
        B, g, V = 8, 7, 20000
        t = make_workload("tree_sample63", B=4, N=15, V=9000, seed=seed)
        self.tree = {k: to_dev(np.ascontiguousarray(t[k])) for k in ("target", "draft", "node_tokens", "parent",
                                                                       "uniforms")}
        self.Tt = float(t["temperature"])
        # EAGLE-style: feature rows through an LM head, then verification
        rng = np.random.default_rng(100 + seed)
        from gen.synth import f32_to_bf16_bits
        eB, eg, ed, eV = 4, 3, 128, 3000
        self.eag = {
            "ft": to_dev(f32_to_bf16_bits(rng.normal(0.0, 1.0, (eB * (eg + 1), ed)).astype(np.float32))),
            "fd": to_dev(f32_to_bf16_bits(rng.normal(0.0, 1.0, (eB * eg, ed)).astype(np.float32))),
            "W": to_dev(f32_to_bf16_bits(rng.normal(0.0, 0.1, (ed, eV)).astype(np.float32))),
            "x": to_dev(rng.integers(0, eV, (eB, eg)).astype(np.int32)),
            "u": to_dev(rng.random((eB, eg + 1), dtype=np.float32)),
        }
        dev = self.lin["target"].device
        i32 = dict(dtype=torch.int32, device=dev)
        self.ws = {m: L.new_workspace(m, *shape, device=dev) for m, shape in (
            (L.MODE_SAMPLE, (B, g, V)), (L.MODE_GREEDY, (B, g, V)), (L.MODE_TREE, (4, 15, 9000)),
            (L.MODE_TREE_SAMPLE, (4, 15, 9000)))}
        self.ws_ee = L.new_workspace(L.MODE_SAMPLE, B, g, V, device=dev)
        self.ws_lm = L.new_workspace(L.MODE_LMHEAD, eB, eg, eV, ed, device=dev)
        self.out = {
            "sample": (torch.empty(B, **i32), torch.empty((B, g + 1), **i32)),
            "early": (torch.empty(B, **i32), torch.empty((B, g + 1), **i32)),
            "greedy": (torch.empty(B, **i32), torch.empty((B, g + 1), **i32)),
            "tree": (torch.empty(4, **i32), torch.empty((4, 15), **i32), torch.empty((4, 15), **i32)),
            "tsample": (torch.empty(4, **i32), torch.empty((4, 15), **i32), torch.empty((4, 15), **i32)),
            "lmhead": (torch.empty(eB, **i32), torch.empty((eB, eg + 1), **i32)),
        }
        self.clear()                             # no output starts from recycled memory

    def run(self):
        a, t = self.lin, self.tree
        L.verify_sample(a["target"], a["draft"], a["draft_tokens"], a["uniforms"], self.T,
                        ws=self.ws[L.MODE_SAMPLE], out=self.out["sample"])
        L.verify_sample(a["target"], a["draft"], a["draft_tokens"], a["uniforms"], self.T, ws=self.ws_ee,
                        out=self.out["early"], early_exit=True)
        L.verify_greedy(a["target"], a["draft_tokens"], ws=self.ws[L.MODE_GREEDY], out=self.out["greedy"])
        L.verify_tree(t["target"], t["node_tokens"], t["parent"], ws=self.ws[L.MODE_TREE], out=self.out["tree"])
        L.verify_tree_sample(t["target"], t["draft"], t["node_tokens"], t["parent"], t["uniforms"], self.Tt,
                             ws=self.ws[L.MODE_TREE_SAMPLE], out=self.out["tsample"])
        e = self.eag
        L.lmhead_verify(e["ft"], e["fd"], e["W"], e["x"], e["u"], 1.0, ws=self.ws_lm, out=self.out["lmhead"])

    def snapshot(self):
        return {k: [x.cpu().numpy().copy() for x in v] for k, v in self.out.items()}

    def clear(self):
        for v in self.out.values():
            for x in v:
                x.fill_(-7)

    def load(self, other):
        """Copy another instance's inputs into this one's buffers."""
        for d, s in ((self.lin, other.lin), (self.tree, other.tree), (self.eag, other.eag)):
            for k in d:
                d[k].copy_(s[k])


def _same(a, b):
    return all(np.array_equal(x, y) for k in a for x, y in zip(a[k], b[k]))


def test_graph_capture_replays_match_eager():
    c = _Calls(seed=1)
    c.run()
    torch.cuda.synchronize()
    want = c.snapshot()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        c.run()                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        c.run()
    for rep in range(3):
        c.clear()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(c.snapshot(), want), rep
        # eager work between the replays
        c.run()
        torch.cuda.synchronize()
        assert _same(c.snapshot(), want), rep
    # new inputs in the captured buffers: the replay reads them
    other = _Calls(seed=2)
    other.run()
    torch.cuda.synchronize()
    want2 = other.snapshot()
    assert not _same(want2, want)
    c.load(other)
    c.clear()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert _same(c.snapshot(), want2)


def test_two_streams_with_separate_workspaces():
    a, b = _Calls(seed=3), _Calls(seed=4)
    a.run()
    b.run()
    torch.cuda.synchronize()
    wa, wb = a.snapshot(), b.snapshot()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(4):
        a.clear()
        b.clear()
        torch.cuda.synchronize()
        for _ in range(3):
            with torch.cuda.stream(sa):
                a.run()
            with torch.cuda.stream(sb):
                b.run()
        torch.cuda.synchronize()
        assert _same(a.snapshot(), wa) and _same(b.snapshot(), wb), rep
