"""spec_verify_sample_noalloc (the allocation-free variant of
spec_verify_sample, whose workspace is the library's static per-GPU scratch
array) against spec_verify_sample with a caller workspace, through the C ABI.

The two must agree bit for bit: the same kernels run on the same workspace
layout.  Calls follow each other on one GPU with shrinking and growing
sizes, so the scratch array always holds the previous call's contents.
"""
import ctypes

import numpy as np
import pytest
import torch

import lossless_draft_verification_03_amd as L
from gen import make_workload
from parity import to_dev
from sentinel import SENT_I32

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _outs(B, g1, dev):
    return (torch.full((B,), SENT_I32, dtype=torch.int32, device=dev),
            torch.full((B, g1), SENT_I32, dtype=torch.int32, device=dev))


def _noalloc(t, d, x, u, T):
    B, g1, V = t.shape
    acc, out = _outs(B, g1, t.device)
    st = L.lib.spec_verify_sample_noalloc(_p(t), _p(d), L.dtype_code(t), _p(x), _p(u), B, g1 - 1, V, float(T),
                                          _p(acc), _p(out),
                                          ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream))
    assert st == L.SPEC_OK, L.lib.spec_status_str(st)
    return acc, out


def _with_workspace(t, d, x, u, T):
    B, g1, V = t.shape
    acc, out = _outs(B, g1, t.device)
    ws = L.new_workspace(L.MODE_SAMPLE, B, g1 - 1, V, device=t.device)
    ws.fill_(0xA5)
    return L.verify_sample(t, d, x, u, T, ws=ws, out=(acc, out))


def _inputs(w):
    return (to_dev(w["target"]), to_dev(w["draft"]), to_dev(w["draft_tokens"]), to_dev(w["uniforms"]),
            float(w["temperature"]))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def test_noalloc_equals_workspace_call_across_sizes():
    big = make_workload("b64g7v128k", cache=True)                                   # B=64, gamma=7, V=128256
    small = make_workload("tiny", B=5, gamma=3, V=3001, dtype="f32", seed=2)       # smaller, ragged V
    mid = make_workload("tiny", B=33, gamma=6, V=20000, dtype="bf16", seed=3)
    for w in (big, small, mid, big):
        args = _inputs(w)
        want = _with_workspace(*args)
        got = _noalloc(*args)
        torch.cuda.synchronize()
        assert torch.equal(got[0], want[0]) and torch.equal(got[1], want[1])
        assert int(got[0].min()) >= 0


def test_noalloc_two_calls_in_a_row_second_smaller():
    a = _inputs(make_workload("b64g7v128k", B=48, V=50000, seed=7))
    b = _inputs(make_workload("tiny", B=3, gamma=2, V=777, dtype="bf16", seed=8))
    wa, wb = _with_workspace(*a), _with_workspace(*b)
    ga = _noalloc(*a)                 # both enqueued before either is read
    gb = _noalloc(*b)
    torch.cuda.synchronize()
    assert torch.equal(ga[0], wa[0]) and torch.equal(ga[1], wa[1])
    assert torch.equal(gb[0], wb[0]) and torch.equal(gb[1], wb[1])


def test_noalloc_rejects_sizes_past_the_scratch_limit():
    t, d, x, u, T = _inputs(make_workload("tiny", B=2, gamma=2, V=64, seed=1))
    acc, out = _outs(2, 3, t.device)
    limit = L.SPEC_NOALLOC_SCRATCH_BYTES
    B = 4096
    assert L.workspace_bytes(L.MODE_SAMPLE, B, 7, 128256) > limit
    st = L.lib.spec_verify_sample_noalloc(_p(t), _p(d), L.SPEC_F32, _p(x), _p(u), B, 7, 128256, 0.7, _p(acc),
                                          _p(out), None)
    assert st == L.SPEC_EWORKSPACE
    torch.cuda.synchronize()
    assert int(acc.min()) == SENT_I32                                               # nothing was launched
