"""HIP graph capture of the forward entry points.

A launch enqueues one kernel and nothing else (no allocation, no memset), so
it can be captured into a graph and replayed. Each test captures one call with
preallocated outputs, then replays the graph several times with new inputs
copied into the captured buffers, with eager work and synchronisation between
the replays, and checks every replay against an eager call on the same inputs:
the kernels are deterministic, so the two agree bit for bit.
"""
import numpy as np
import pytest
import torch

import exact_attention_16_amd as fa
import workloads as W
from gpu_util import device

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _banner(msg):
    print(msg, flush=True)


def _capture(fn):
    # warm up on a side stream first, as torch asks before a capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_check(g, inputs, outputs, eager, fresh, tag):
    for r in range(REPLAYS):
        for t, x in zip(inputs, fresh(r)):
            t.copy_(x)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = eager()
        torch.cuda.synchronize()
        for got, want in zip(outputs, ref):
            assert torch.equal(got, want), f"{tag}: replay {r} differs from the eager call"
        _banner(f"{tag}: replay {r} bitwise-equal to eager")


@pytest.mark.parametrize("D,dtype,causal", [(128, torch.bfloat16, True), (64, torch.float16, False)])
def test_graph_dense(D, dtype, causal):
    B, H, S = 2, 4, 1000
    tag = f"graph dense B={B} H={H} S={S} D={D} {dtype} causal={causal}"
    _banner(tag)
    dev = device()
    gen = torch.Generator().manual_seed(9000 + D)
    mk = lambda: torch.randn(B, H, S, D, generator=gen).to(dtype).to(dev)
    q, k, v = mk(), mk(), mk()
    o = torch.empty_like(q)
    lse = torch.empty(B, H, S, dtype=torch.float32, device=dev)
    g = _capture(lambda: fa.attention(q, k, v, causal, out=o, lse=lse))
    _replay_and_check(g, (q, k, v), (o, lse), lambda: fa.attention(q, k, v, causal),
                      lambda r: (mk(), mk(), mk()), tag)


def test_graph_varlen():
    H, D = 8, 128
    lengths = [300, 0, 1025, 77, 512]
    tag = f"graph varlen H={H} D={D} lengths={lengths}"
    _banner(tag)
    dev = device()
    total = sum(lengths)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=dev)
    gen = torch.Generator().manual_seed(9100)
    mk = lambda: torch.randn(total, H, D, generator=gen).to(torch.bfloat16).to(dev)
    q, k, v = mk(), mk(), mk()
    o = torch.empty_like(q)
    lse = torch.empty(H, total, dtype=torch.float32, device=dev)
    L = max(lengths)
    g = _capture(lambda: fa.attention_varlen(q, k, v, cu, cu, L, L, True, out=o, lse=lse))
    _replay_and_check(g, (q, k, v), (o, lse),
                      lambda: fa.attention_varlen(q, k, v, cu, cu, L, L, True),
                      lambda r: (mk(), mk(), mk()), tag)


def test_graph_fp8():
    B, H, S, D = 1, 4, 700, 128
    tag = f"graph fp8 B={B} H={H} S={S} D={D}"
    _banner(tag)
    dev = device()
    rng = np.random.default_rng(9200)

    def mk():
        codes, ds = W.quantize_e4m3(rng.standard_normal((B, H, S, D)).astype(np.float32))
        return torch.from_numpy(np.ascontiguousarray(codes)).to(dev), ds

    (q, dq), (k, dk), (v, dv) = mk(), mk(), mk()
    o = torch.empty(B, H, S, D, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, H, S, dtype=torch.float32, device=dev)
    # the descales are launch arguments, fixed at capture: new inputs keep them
    g = _capture(lambda: fa.attention_fp8(q, k, v, dq, dk, dv, True, out=o, lse=lse))

    def fresh(r):
        return tuple(mk()[0] for _ in range(3))

    _replay_and_check(g, (q, k, v), (o, lse),
                      lambda: fa.attention_fp8(q, k, v, dq, dk, dv, True), fresh, tag)
