"""GPU parity for the strided and variable-length entry points against the
float64 oracle: query and key lengths that differ (causal mask aligned
bottom-right), [B, S, H, D] and other strided layouts, a key/value head shared
by every query head, and sequences of different lengths packed along a token
axis. Same tolerances as the dense path.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_16_amd as fa
import oracle
import workloads as W
from gpu_util import LSE_TOL, O_TOL, TORCH_DT, device, o_to_f64, to_dev

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(msg, flush=True)


def _assert_close(og, lg, o_ref, l_ref, dtype, tag):
    """O within the dtype's tolerance; lse within LSE_TOL where finite, and -inf
    exactly where the oracle has -inf (rows that see no key)."""
    assert np.all(np.isfinite(og)), tag
    eo = float(np.abs(og - o_ref).max()) if og.size else 0.0
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isneginf(lg), ~fin), (tag, "rows without keys")
    el = float(np.abs(lg[fin] - l_ref[fin]).max()) if fin.any() else 0.0
    _banner(f"{tag}: max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= O_TOL[dtype], (tag, eo)
    assert el <= LSE_TOL, (tag, el)


def _bits(shape, dtype, seed):
    return W.random_bits(shape, dtype, seed)


# ------------------------------------------------ query and key lengths differ

@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,Sk", [(256, 512), (512, 256), (100, 300), (300, 100), (1, 700),
                                   (700, 1), (97, 96)])
def test_two_lengths_all_rows(Sq, Sk, causal, D, dtype):
    tag = f"Sq={Sq} Sk={Sk} causal={causal} D={D} {dtype}"
    _banner(tag)
    seed = 5000 + Sq + 3 * Sk + D + causal
    qb, kb, vb = _bits((1, 2, Sq, D), dtype, seed), _bits((1, 2, Sk, D), dtype, seed + 1), \
        _bits((1, 2, Sk, D), dtype, seed + 2)
    q, k, v = to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype)
    o, lse = fa.attention(q, k, v, causal)
    torch.cuda.synchronize()
    scale = float(np.float32(1.0 / math.sqrt(D)))
    o_ref, l_ref = oracle.attention_fwd(W.decode(qb, dtype), W.decode(kb, dtype),
                                        W.decode(vb, dtype), causal, scale)
    _assert_close(o_to_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, dtype, tag)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,Sk", [(1024, 1536), (1536, 1024)])
def test_two_lengths_eight_wave_kernel(Sq, Sk, causal):
    """Enough work-groups for the ping-pong kernel; sampled heads, every row."""
    dtype, D, H = W.BF16, 128, 64
    tag = f"pp Sq={Sq} Sk={Sk} causal={causal}"
    _banner(tag)
    assert fa.fa_fwd_tile(D, 1, H, Sq)[2] == 512
    qb, kb, vb = _bits((1, H, Sq, D), dtype, 61), _bits((1, H, Sk, D), dtype, 62), \
        _bits((1, H, Sk, D), dtype, 63)
    o, lse = fa.attention(to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype), causal)
    torch.cuda.synchronize()
    og, lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    for h in (0, 17, 63):
        o_ref, l_ref = oracle.attention_fwd(W.decode(qb[0, h], dtype), W.decode(kb[0, h], dtype),
                                            W.decode(vb[0, h], dtype), causal, scale)
        _assert_close(og[0, h], lg[0, h], o_ref, l_ref, dtype, f"{tag} h={h}")


def test_no_keys_gives_zero_rows():
    """Sk = 0: every row sees no key, so O = 0 and lse = -inf (raw C call with
    real allocations, since an empty torch tensor may have no address)."""
    dtype, D = W.F16, 64
    _banner("Sk=0")
    q = to_dev(_bits((1, 1, 64, D), dtype, 70), dtype)
    kv = torch.zeros((1, 1, 8, D), dtype=torch.float16, device=device())
    o = torch.full_like(q, 7.0)
    lse = torch.zeros((1, 1, 64), dtype=torch.float32, device=device())
    st = [64 * D, 64 * D, D, 8 * D, 8 * D, D, 8 * D, 8 * D, D, 64 * D, 64 * D, D, 64, 64]
    for causal in (0, 1):
        fa.fa_fwd_strided(q.data_ptr(), kv.data_ptr(), kv.data_ptr(), o.data_ptr(),
                          lse.data_ptr(), 1, 1, 64, 0, D, causal, 0.125,
                          torch.cuda.current_stream().cuda_stream, W.DTYPE_CODE[dtype], st)
        torch.cuda.synchronize()
        assert torch.all(o == 0) and torch.all(torch.isneginf(lse)), causal


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_huge_output_row_stride(causal, D):
    """One query row and an output row stride of 2^29 elements (2^30 bytes,
    inside the per-head limit): the kernel's padding rows past the last query
    row would land at byte offsets that are multiples of 2^30, which wrap to
    row 0 in 32-bit arithmetic; they must be dropped, so row 0 keeps its own
    result (O's buffer holds just that row)."""
    dtype, Sk = W.BF16, 40
    tag = f"row stride 2^29 causal={causal} D={D}"
    _banner(tag)
    qb, kb, vb = _bits((1, 1, 1, D), dtype, 90 + D), _bits((1, 1, Sk, D), dtype, 91 + D), \
        _bits((1, 1, Sk, D), dtype, 92 + D)
    q, k, v = to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype)
    o = torch.full((D,), 3.0, dtype=torch.bfloat16, device=device())
    lse = torch.zeros((1,), dtype=torch.float32, device=device())
    st = [D, D, D, Sk * D, Sk * D, D, Sk * D, Sk * D, D, D, D, 1 << 29, 1, 1]
    scale = float(np.float32(1.0 / math.sqrt(D)))
    fa.fa_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      1, 1, 1, Sk, D, causal, scale, torch.cuda.current_stream().cuda_stream,
                      W.DTYPE_CODE[dtype], st)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_fwd(W.decode(qb, dtype), W.decode(kb, dtype),
                                        W.decode(vb, dtype), causal, scale)
    _assert_close(o_to_f64(o.view(1, 1, 1, D)), lse.cpu().numpy().astype(np.float64).reshape(1, 1, 1),
                  o_ref, l_ref, dtype, tag)


# ------------------------------------------------------------ strided layouts

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_bshd_layout(causal, D):
    dtype, B, H, Sq, Sk = W.BF16, 2, 3, 200, 333
    tag = f"bshd causal={causal} D={D}"
    _banner(tag)
    qb, kb, vb = _bits((B, Sq, H, D), dtype, 80 + D), _bits((B, Sk, H, D), dtype, 81 + D), \
        _bits((B, Sk, H, D), dtype, 82 + D)
    o, lse = fa.attention(to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype), causal,
                          layout="bshd")
    torch.cuda.synchronize()
    assert o.shape == (B, Sq, H, D) and lse.shape == (B, H, Sq)
    tr = lambda x: W.decode(x, dtype).transpose(0, 2, 1, 3)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    o_ref, l_ref = oracle.attention_fwd(tr(qb), tr(kb), tr(vb), causal, scale)
    _assert_close(o_to_f64(o).transpose(0, 2, 1, 3), lse.cpu().numpy().astype(np.float64),
                  o_ref, l_ref, dtype, tag)


@pytest.mark.parametrize("causal", [False, True])
def test_row_stride_views_in_and_out(causal):
    """q, k, v and o are views with rows wider than D (row stride 2D)."""
    dtype, B, H, S, D = W.F16, 2, 2, 300, 64
    tag = f"views causal={causal}"
    _banner(tag)
    wide = [_bits((B, H, S, 2 * D), dtype, 90 + i) for i in range(3)]
    q, k, v = (to_dev(x, dtype)[..., :D] for x in wide)
    big_o = torch.zeros((B, H, S, 2 * D), dtype=torch.float16, device=device())
    out = big_o[..., D:]
    _o, lse = fa.attention(q, k, v, causal, out=out)
    torch.cuda.synchronize()
    assert torch.all(big_o[..., :D] == 0), "bytes outside the output view written"
    dec = [W.decode(x[..., :D], dtype) for x in wide]
    o_ref, l_ref = oracle.attention_fwd(*dec, causal, float(np.float32(1.0 / math.sqrt(D))))
    _assert_close(o_to_f64(out), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, dtype, tag)


@pytest.mark.parametrize("causal", [False, True])
def test_one_kv_head_shared_by_all_query_heads(causal):
    """k and v with head stride 0 (one key/value head broadcast to H query heads)."""
    dtype, B, H, S, D = W.BF16, 1, 8, 257, 128
    tag = f"shared kv head causal={causal}"
    _banner(tag)
    qb = _bits((B, H, S, D), dtype, 100)
    kb, vb = _bits((B, 1, S, D), dtype, 101), _bits((B, 1, S, D), dtype, 102)
    k = to_dev(kb, dtype).expand(B, H, S, D)
    v = to_dev(vb, dtype).expand(B, H, S, D)
    assert k.stride(1) == 0
    o, lse = fa.attention(to_dev(qb, dtype), k, v, causal)
    torch.cuda.synchronize()
    rep = lambda x: np.repeat(W.decode(x, dtype), H, axis=1)
    o_ref, l_ref = oracle.attention_fwd(W.decode(qb, dtype), rep(kb), rep(vb), causal,
                                        float(np.float32(1.0 / math.sqrt(D))))
    _assert_close(o_to_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, dtype, tag)


# ----------------------------------------------------- variable-length batches

def _varlen_inputs(lq, lk, H, D, dtype, seed):
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    qb = _bits((int(cq[-1]), H, D), dtype, seed)
    kb = _bits((int(ck[-1]), H, D), dtype, seed + 1)
    vb = _bits((int(ck[-1]), H, D), dtype, seed + 2)
    return cq, ck, qb, kb, vb


def _run_varlen(cq, ck, qb, kb, vb, dtype, causal, lq, lk):
    cu_q = torch.from_numpy(cq).to(device())
    cu_k = torch.from_numpy(ck).to(device())
    o, lse = fa.attention_varlen(to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype), cu_q,
                                 cu_k, max(lq), max(lk), causal)
    torch.cuda.synchronize()
    return o_to_f64(o), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_all_rows(causal, D, dtype):
    lq = [0, 1, 77, 256, 300, 513, 64]
    lk = [3, 1, 77, 512, 100, 513, 0]
    H = 3
    tag = f"varlen causal={causal} D={D} {dtype}"
    _banner(tag)
    cq, ck, qb, kb, vb = _varlen_inputs(lq, lk, H, D, dtype, 110 + D + causal)
    og, lg = _run_varlen(cq, ck, qb, kb, vb, dtype, causal, lq, lk)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    o_ref, l_ref = oracle.attention_varlen(W.decode(qb, dtype), W.decode(kb, dtype),
                                           W.decode(vb, dtype), cq, ck, causal, scale)
    _assert_close(og, lg, o_ref, l_ref, dtype, tag)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_eight_wave_kernel(causal):
    """A batch with enough work-groups for the ping-pong kernel; sampled
    (sequence, head) pairs, every row of each."""
    dtype, D, H = W.BF16, 128, 32
    rng = np.random.default_rng(120)
    lq = [int(x) for x in rng.integers(200, 1025, size=8)]
    lk = [x + int(d) for x, d in zip(lq, rng.integers(-150, 151, size=8))]
    tag = f"varlen pp causal={causal}"
    _banner(tag)
    assert fa.fa_fwd_tile(D, len(lq), H, max(lq))[2] == 512
    cq, ck, qb, kb, vb = _varlen_inputs(lq, lk, H, D, dtype, 121)
    og, lg = _run_varlen(cq, ck, qb, kb, vb, dtype, causal, lq, lk)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    for b, h in ((0, 0), (3, 31), (7, 5)):
        qs, ks = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        o_ref, l_ref = oracle.attention_fwd(W.decode(qb[qs, h], dtype), W.decode(kb[ks, h], dtype),
                                            W.decode(vb[ks, h], dtype), causal, scale)
        _assert_close(og[qs, h], lg[h, qs], o_ref, l_ref, dtype, f"{tag} b={b} h={h}")


@pytest.mark.parametrize("H", [2, 96])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_sequences_past_the_maxima_are_marked(causal, D, H):
    """A sequence longer than max_seqlen_q, or with more keys than
    max_seqlen_k, is not computed: all its rows get NaN in O and lse; every
    other sequence is exact. (H = 2 runs the small-grid kernels, H = 96 the
    256-row ones.)"""
    dtype = W.BF16
    scale = float(np.float32(1.0 / math.sqrt(D)))
    # (query lengths, key lengths, max_q, max_k, sequences past a maximum)
    cases = [([40, 300, 60], [40, 100, 60], 256, 100, [1]),        # queries past max_q
             ([40, 90, 60], [40, 90, 200], 128, 128, [2]),         # keys past max_k
             ([300, 50, 260], [30, 300, 260], 256, 256, [0, 1, 2])]  # both, every sequence
    for n, (lq, lk, max_q, max_k, cut) in enumerate(cases):
        _banner(f"varlen past the maxima causal={causal} D={D} H={H} case {n}")
        cq, ck, qb, kb, vb = _varlen_inputs(lq, lk, H, D, dtype, 150 + 10 * n + D + H)
        cu_q = torch.from_numpy(cq).to(device())
        cu_k = torch.from_numpy(ck).to(device())
        o, lse = fa.attention_varlen(to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype),
                                     cu_q, cu_k, max_q, max_k, causal)
        torch.cuda.synchronize()
        og, lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
        bad = np.zeros(int(cq[-1]), dtype=bool)
        for b in cut:
            bad[cq[b]:cq[b + 1]] = True
        assert np.all(np.isnan(og[bad])) and np.all(np.isnan(lg[:, bad])), "cut rows not marked"
        if (~bad).any():
            o_ref, l_ref = oracle.attention_varlen(W.decode(qb, dtype), W.decode(kb, dtype),
                                                   W.decode(vb, dtype), cq, ck, causal, scale)
            _assert_close(og[~bad], lg[:, ~bad], o_ref[~bad], l_ref[:, ~bad], dtype,
                          f"varlen rows within the maxima, case {n}")


def test_varlen_offsets_past_the_tensors_are_clamped():
    """The last sequence's end offset lies past total_q / total_k: the kernel
    clamps it to the tensors (the sequence ends at the last token row) and
    every other sequence is unaffected."""
    dtype, D, H = W.F16, 64, 2
    lq, lk = [40, 90, 60], [40, 90, 60]
    _banner("varlen clamped offsets")
    cq, ck, qb, kb, vb = _varlen_inputs(lq, lk, H, D, dtype, 130)
    cq_bad, ck_bad = cq.copy(), ck.copy()
    cq_bad[-1] += 1000
    ck_bad[-1] += 1000
    cu_q = torch.from_numpy(cq_bad).to(device())
    cu_k = torch.from_numpy(ck_bad).to(device())
    o, lse = fa.attention_varlen(to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype), cu_q,
                                 cu_k, 1100, 1100, True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_varlen(W.decode(qb, dtype), W.decode(kb, dtype),
                                           W.decode(vb, dtype), cq, ck, True,
                                           float(np.float32(1.0 / math.sqrt(D))))
    _assert_close(o_to_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, dtype,
                  "varlen clamped")


# A variable-length launch of at most 256 sequences runs only the query tiles
# within the sequences (each work-group finds its tile from the offsets); a
# larger batch runs the full grid. The outputs start as NaN, so a row that no
# work-group writes fails the comparison.

def _run_varlen_prefilled(cq, ck, qb, kb, vb, dtype, causal, max_q, max_k):
    dev = device()
    H, D = qb.shape[1], qb.shape[2]
    out = torch.full(qb.shape, float("nan"), dtype=TORCH_DT[dtype], device=dev)
    lse = torch.full((H, qb.shape[0]), float("nan"), dtype=torch.float32, device=dev)
    cu_q = torch.from_numpy(cq).to(dev)
    cu_k = torch.from_numpy(ck).to(dev)
    fa.attention_varlen(to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype), cu_q, cu_k,
                        max_q, max_k, causal, out=out, lse=lse)
    torch.cuda.synchronize()
    return o_to_f64(out), lse.cpu().numpy().astype(np.float64)


def _skewed_lengths(rng, B, short, long_lens):
    """B sequences: short ones (0 .. short-1 tokens, some empty) with the long
    ones placed among them."""
    L = [int(x) for x in rng.integers(0, short, size=B - len(long_lens))]
    for n, x in enumerate(long_lens):
        L.insert((n + 1) * len(L) // (len(long_lens) + 1), x)
    return L


@pytest.mark.parametrize("H", [3, 8])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_compacted_launch_all_rows(causal, D, H):
    """One long sequence among 40 short or empty ones: the full grid would be
    mostly query tiles past the sequences' ends. H = 8 takes the XCD order
    (heads x, x+8, ... of each sequence per XCD), H = 3 the plain one."""
    dtype = W.BF16
    rng = np.random.default_rng(200 + D + H + causal)
    lq = _skewed_lengths(rng, 41, 120, [2048])
    lk = list(lq)
    tag = f"varlen compacted causal={causal} D={D} H={H}"
    _banner(tag)
    cq, ck, qb, kb, vb = _varlen_inputs(lq, lk, H, D, dtype, 210 + D + H)
    og, lg = _run_varlen_prefilled(cq, ck, qb, kb, vb, dtype, causal, max(lq), max(lk))
    o_ref, l_ref = oracle.attention_varlen(W.decode(qb, dtype), W.decode(kb, dtype),
                                           W.decode(vb, dtype), cq, ck, causal,
                                           float(np.float32(1.0 / math.sqrt(D))))
    _assert_close(og, lg, o_ref, l_ref, dtype, tag)


@pytest.mark.parametrize("B,H,causal", [(200, 8, True), (256, 2, False), (300, 2, True)])
def test_varlen_many_sequences_all_rows(B, H, causal):
    """200 and 256 sequences span many lanes of the work-groups' offset scan
    (four sequences per lane); 300 is past the compacted launch's limit and
    runs the full grid."""
    dtype, D = W.F16, 64
    rng = np.random.default_rng(230 + B)
    lq = _skewed_lengths(rng, B, 90, [700, 1300])
    lk = [max(0, x + int(d)) for x, d in zip(lq, rng.integers(-20, 21, size=B))]
    tag = f"varlen B={B} H={H} causal={causal}"
    _banner(tag)
    cq, ck, qb, kb, vb = _varlen_inputs(lq, lk, H, D, dtype, 240 + B)
    og, lg = _run_varlen_prefilled(cq, ck, qb, kb, vb, dtype, causal, max(lq), max(lk))
    o_ref, l_ref = oracle.attention_varlen(W.decode(qb, dtype), W.decode(kb, dtype),
                                           W.decode(vb, dtype), cq, ck, causal,
                                           float(np.float32(1.0 / math.sqrt(D))))
    _assert_close(og, lg, o_ref, l_ref, dtype, tag)


@pytest.mark.parametrize("H", [2, 64])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_decreasing_offsets_mark_every_row(causal, D, H):
    """Offsets that decrease, against the stated order, in a compacted launch:
    no sequence is computed and every row of O and lse is NaN. (H = 2 runs
    the four-wave kernel at D = 128 and the key-split kernel at D = 64, H = 64
    the 256-row kernels.)"""
    dtype = W.BF16
    _banner(f"varlen decreasing offsets causal={causal} D={D} H={H}")
    cq = np.array([0, 100, 50, 200, 400], dtype=np.int32)
    ck = np.array([0, 100, 150, 200, 400], dtype=np.int32)
    qb = _bits((400, H, D), dtype, 260)
    kb = _bits((400, H, D), dtype, 261)
    vb = _bits((400, H, D), dtype, 262)
    og, lg = _run_varlen_prefilled(cq, ck, qb, kb, vb, dtype, causal, 2000, 2000)
    assert np.all(np.isnan(og)) and np.all(np.isnan(lg))
    # the same offsets in order compute every row
    cq_ok = np.array([0, 50, 100, 200, 400], dtype=np.int32)
    og, lg = _run_varlen_prefilled(cq_ok, ck, qb, kb, vb, dtype, causal, 2000, 2000)
    o_ref, l_ref = oracle.attention_varlen(W.decode(qb, dtype), W.decode(kb, dtype),
                                           W.decode(vb, dtype), cq_ok, ck, causal,
                                           float(np.float32(1.0 / math.sqrt(D))))
    _assert_close(og, lg, o_ref, l_ref, dtype, f"varlen ordered offsets causal={causal} D={D} H={H}")


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_partial_final_tiles_all_rows(causal):
    """Sixteen sequences whose last 256-row query tile holds 1-128 rows: in
    those tiles the second group of four waves has no rows and only takes its
    share of the K/V loads and barriers. Every row of the ping-pong kernel's
    result against the oracle, outputs filled with NaN first."""
    dtype, D, H = W.BF16, 128, 8
    rng = np.random.default_rng(270 + causal)
    lq = [256 * int(m) + int(r) for m, r in zip(rng.integers(0, 4, size=16), rng.integers(1, 129, size=16))]
    lk = list(lq)
    assert fa.fa_fwd_tile(D, len(lq), H, max(lq))[2] == 512
    tag = f"varlen partial final tiles causal={causal}"
    _banner(tag)
    cq, ck, qb, kb, vb = _varlen_inputs(lq, lk, H, D, dtype, 280 + causal)
    og, lg = _run_varlen_prefilled(cq, ck, qb, kb, vb, dtype, causal, max(lq), max(lk))
    o_ref, l_ref = oracle.attention_varlen(W.decode(qb, dtype), W.decode(kb, dtype),
                                           W.decode(vb, dtype), cq, ck, causal,
                                           float(np.float32(1.0 / math.sqrt(D))))
    _assert_close(og, lg, o_ref, l_ref, dtype, tag)
