"""Repeated launches of each kernel on the same inputs return bitwise-identical
O and lse. A timing-dependent hazard (a race between one work-group's loads
and another's reads, a store reading its data registers late) shows up as a
difference between launches. The configurations keep work-groups out of
step: partial final query tiles in which some waves have no rows, many
sequences of different lengths, grids with more than one work-group per CU.
Outputs start as NaN, so a row no launch writes fails too. (Such a hazard
was found this way: 16-byte O stores whose data registers the next
instruction had overwritten, in a few rows of some launches.)
"""
import numpy as np
import pytest
import torch

import exact_attention_16_amd as fa
import workloads as W
from gpu_util import TORCH_DT, device, to_dev

pytestmark = pytest.mark.gpu

LAUNCHES = 4


def _banner(msg):
    print(msg, flush=True)


def _same_every_launch(run, tag):
    first = None
    for n in range(LAUNCHES):
        o, lse = run()
        torch.cuda.synchronize()
        assert not torch.isnan(o.float()).any(), f"{tag}: O not written (launch {n})"
        assert not torch.isnan(lse).any(), f"{tag}: lse not written (launch {n})"
        if first is None:
            first = (o.clone(), lse.clone())
        else:
            assert torch.equal(o, first[0]) and torch.equal(lse, first[1]), \
                f"{tag}: launch {n} differs from launch 0"
    _banner(f"{tag}: {LAUNCHES} launches bitwise equal")


def _mixed_lengths(seed, B):
    """B sequences whose final 256-row query tile holds 1..255 rows."""
    rng = np.random.default_rng(seed)
    return [256 * int(m) + int(r) for m, r in zip(rng.integers(0, 6, size=B),
                                                  rng.integers(1, 256, size=B))]


@pytest.mark.parametrize("D,H,causal,dtype,threads", [(128, 8, True, W.BF16, 512),
                                                      (64, 16, False, W.F16, 512)])
def test_varlen_repeat_launches(D, H, causal, dtype, threads):
    """48 sequences: the ping-pong kernel (D = 128, causal) and the
    four-waves-per-SIMD kernel (D = 64)."""
    L = _mixed_lengths(300 + D, 48)
    assert fa.fa_fwd_tile(D, len(L), H, max(L), causal)[2] == threads
    cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    total = int(cu[-1])
    q, k, v = (to_dev(W.random_bits((total, H, D), dtype, 310 + i), dtype) for i in range(3))
    cud = torch.from_numpy(cu).to(device())
    out = torch.empty_like(q)
    lse = torch.empty((H, total), dtype=torch.float32, device=device())

    def run():
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        return fa.attention_varlen(q, k, v, cud, cud, max(L), max(L), causal, out=out, lse=lse)

    _same_every_launch(run, f"varlen D={D} H={H} causal={causal}")


@pytest.mark.parametrize("B,H,S,D,causal,dtype", [
    (1, 63, 1024, 128, True, W.BF16),   # four-wave kernel, 504 work-groups
    (1, 16, 1024, 64, True, W.F16),     # key-split kernel
    (4, 16, 200, 64, False, W.F16),     # four-wave kernel at D = 64, ragged S
    (2, 16, 2900, 128, True, W.BF16),   # ping-pong kernel, partial final tile
])
def test_dense_repeat_launches(B, H, S, D, causal, dtype):
    q, k, v = (to_dev(W.random_bits((B, H, S, D), dtype, 320 + i), dtype) for i in range(3))
    out = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=device())

    def run():
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        return fa.attention(q, k, v, causal, out=out, lse=lse)

    _same_every_launch(run, f"dense B={B} H={H} S={S} D={D} causal={causal}")


@pytest.mark.parametrize("S,D,causal", [(2900, 128, True), (1000, 64, False)])
def test_fp8_repeat_launches(S, D, causal):
    """The 8-bit kernel, partial final tile."""
    B, H = 1, 16
    rng = np.random.default_rng(330 + D)
    enc = [W.quantize_e4m3(rng.standard_normal((B, H, S, D)).astype(np.float32)) for _ in range(3)]
    q, k, v = (torch.from_numpy(np.ascontiguousarray(c)).to(device()) for c, _ in enc)
    ds = [d for _, d in enc]
    out = torch.empty((B, H, S, D), dtype=TORCH_DT[W.BF16], device=device())
    lse = torch.empty((B, H, S), dtype=torch.float32, device=device())

    def run():
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        return fa.attention_fp8(q, k, v, ds[0], ds[1], ds[2], causal, out=out, lse=lse)

    _same_every_launch(run, f"fp8 S={S} D={D} causal={causal}")
