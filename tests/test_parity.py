"""GPU parity: the HIP path (through the C ABI) against the float64 CPU oracle
on the same seeded 16-bit inputs.

Tolerance: max |O_gpu - O_oracle| <= 5e-3 (fp16) / 2e-2 (bf16) over every
compared element, and max |lse_gpu - lse_oracle| <= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_16_amd as fa
import oracle
import workloads as W
import diag
from gpu_util import (LSE_TOL, O_TOL, compare_rows, max_abs_err, o_to_f64, run, sample_rows,
                      to_dev, device)

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(msg, flush=True)


VARIANTS = {"k4": diag.VARIANT_FOUR_WAVE, "pp": diag.VARIANT_PING_PONG,
            "ps": diag.VARIANT_PERSISTENT, "sp": diag.VARIANT_SPLIT, "o4": diag.VARIANT_OCC4}
# kernels that exist at D = 64 only
D64_ONLY = ("sp", "o4")


def _exists(kernel, D):
    return D == 64 or kernel not in D64_ONLY


def _skip_absent(kernel, D):
    """The key-split and four-waves-per-SIMD kernels exist at D = 64 only."""
    if not _exists(kernel, D):
        pytest.skip(f"kernel {kernel} runs at D = 64 only")


def _auto_kernel(D, B, H, S, causal):
    """The kernel fa_fwd picks for this shape, by its query rows per
    work-group and keys per tile."""
    bm, bn = fa.fa_fwd_tile(D, B, H, S, causal)[:2]
    if bm == 256 and bn == 64:
        return "o4"
    return {256: "pp", 128: "k4", 64: "sp"}[bm]


def _check_full(qb, kb, vb, dtype, causal, scale, tag, variant=None):
    o, lse = run(qb, kb, vb, dtype, causal, scale, variant=variant)
    og, lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    B, H, S, _ = qb.shape
    eo, el = compare_rows(qb, kb, vb, dtype, causal, scale, og, lg,
                          [((b, h), np.arange(S)) for b in range(B) for h in range(H)])
    _banner(f"{tag}: max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    assert eo <= O_TOL[dtype], (tag, eo)
    assert el <= LSE_TOL, (tag, el)
    return og, lg


@pytest.mark.parametrize("causal", [False, True])
def test_tiny_workload(causal):
    w = W.WORKLOADS["tiny"].with_causal(causal)
    _banner(f"tiny causal={causal}")
    _check_full(*W.make_inputs(w), w.dtype, causal, w.scale, f"tiny causal={causal}")


@pytest.mark.parametrize("kernel", sorted(VARIANTS))
@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [1, 7, 64, 129, 300])
def test_small_shapes_all_rows(S, causal, D, dtype, kernel):
    """Several Q and KV tiles, ragged tails, tiny S; every output compared;
    each shape through every kernel."""
    _skip_absent(kernel, D)
    shape = (2, 3, S, D)
    seed = 1000 + S * 4 + D + (dtype == W.BF16) * 2 + causal
    qb, kb, vb = (W.random_bits(shape, dtype, seed + i) for i in range(3))
    _check_full(qb, kb, vb, dtype, causal, 1.0 / math.sqrt(D),
                f"S={S} D={D} {dtype} causal={causal} kernel={kernel}", VARIANTS[kernel])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
def test_key_split_long_rows_all_rows(dtype, causal):
    """The key-split kernel at S = 1024 (16 KV tiles, four per group, the
    last group's last tile on the causal diagonal): every output compared."""
    S, D = 1024, 64
    qb, kb, vb = (W.random_bits((1, 2, S, D), dtype, 2100 + causal + i) for i in range(3))
    _check_full(qb, kb, vb, dtype, causal, 1.0 / math.sqrt(D),
                f"key split S={S} {dtype} causal={causal}", VARIANTS["sp"])


@pytest.mark.parametrize("kernel", sorted(VARIANTS))
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_many_tiles_all_rows(causal, D, kernel):
    """Many KV tiles per work-group (every stage of both pipelines reused
    several times, the three-stage ring wrapping), a ragged end, all rows."""
    _skip_absent(kernel, D)
    S, dt = 1500, W.BF16
    shape = (1, 2, S, D)
    qb, kb, vb = (W.random_bits(shape, dt, 2000 + D + causal + i) for i in range(3))
    _check_full(qb, kb, vb, dt, causal, 1.0 / math.sqrt(D),
                f"many tiles S={S} D={D} causal={causal} kernel={kernel}", VARIANTS[kernel])


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
def test_four_wave_d128_many_work_groups_all_rows(dtype):
    """B=1 H=63 S=1024 D=128 causal: 504 four-wave work-groups, one per CU,
    their DMA traffic overlapping other work-groups' epilogues. Before the
    epilogue packed every value ahead of its stores, a 16-byte O store read
    its data registers after the next instruction had overwritten them in a
    few rows of every launch of this grid (run two work-groups to a CU). All
    rows of every head, three launches, bitwise equal."""
    B, H, S, D = 1, 63, 1024, 128
    assert _auto_kernel(D, B, H, S, True) == "k4"
    qb, kb, vb = (W.random_bits((B, H, S, D), dtype, 7100 + i) for i in range(3))
    first = None
    for rep in range(3):
        og, lg = _check_full(qb, kb, vb, dtype, True, D ** -0.5,
                             f"four-wave D=128 H=63 {dtype} launch {rep}")
        if first is None:
            first = (og, lg)
        else:
            assert np.array_equal(og, first[0]) and np.array_equal(lg, first[1])


@pytest.mark.parametrize("D", [64, 128])
def test_kernels_agree(D):
    """Both kernels on one input: each within tolerance of the oracle and of
    each other (they differ only in tile sizes, hence rescale points)."""
    S, dt = 777, W.F16
    qb, kb, vb = (W.random_bits((2, 2, S, D), dt, 3000 + D + i) for i in range(3))
    res = [_check_full(qb, kb, vb, dt, True, D ** -0.5, f"agree D={D} {k}", VARIANTS[k])
           for k in sorted(VARIANTS) if _exists(k, D)]
    for other in res[1:]:
        assert np.abs(res[0][0] - other[0]).max() <= O_TOL[dt]
        assert np.abs(res[0][1] - other[1]).max() <= LSE_TOL


# full-size workloads, sampled rows (the oracle computes each row on its own)
_SAMPLES = {"dec": (None, None), "bat": (8, 24), "long": (None, 96), "ramp": (None, 96)}


@pytest.mark.parametrize("name", ["dec", "bat", "long", "ramp"])
def test_workload_full_size(name):
    w = W.WORKLOADS[name]
    _banner(f"workload {name}: B={w.B} H={w.H} S={w.S} D={w.D} {w.dtype} causal={w.causal}")
    qb, kb, vb = W.make_inputs(w)
    o, lse = run(qb, kb, vb, w.dtype, w.causal, w.scale)
    og, lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    full_heads, nrows = _SAMPLES[name]
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    plan = []
    for n, bh in enumerate(heads):
        if nrows is None or (full_heads is not None and n % max(1, len(heads) // full_heads) == 0):
            plan.append((bh, np.arange(w.S)))
        else:
            plan.append((bh, sample_rows(w.S, nrows, seed=n)))
    eo, el = compare_rows(qb, kb, vb, w.dtype, w.causal, w.scale, og, lg, plan)
    _banner(f"workload {name}: rows compared={sum(len(r) for _, r in plan)} "
            f"max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= O_TOL[w.dtype] and el <= LSE_TOL


def test_long_context_max_rows():
    """One head at S=65536 (the largest size tested), causal bf16, sampled rows."""
    shape, dt = (1, 1, 65536, 128), W.BF16
    qb, kb, vb = (W.random_bits(shape, dt, 77 + i) for i in range(3))
    o, lse = run(qb, kb, vb, dt, True, 128 ** -0.5)
    og, lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    eo, el = compare_rows(qb, kb, vb, dt, True, 128 ** -0.5, og, lg,
                          [((0, 0), sample_rows(65536, 48, seed=5))])
    _banner(f"S=65536: max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= O_TOL[dt] and el <= LSE_TOL


def test_two_million_rows():
    """One head at S = 2^21 (a head's K, V and O span 2^29 bytes, a quarter of
    the 32-bit offset range), causal bf16, sampled rows near both ends."""
    S, dt = 1 << 21, W.BF16
    _banner(f"S={S}")
    qb, kb, vb = (W.random_bits((1, 1, S, 128), dt, 88 + i) for i in range(3))
    o, lse = run(qb, kb, vb, dt, True, 128 ** -0.5)
    og, lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(lg).all()
    rows = np.array([0, 1, 255, 256, S // 2 + 7, S - 257, S - 256, S - 2, S - 1])
    eo, el = compare_rows(qb, kb, vb, dt, True, 128 ** -0.5, og, lg, [((0, 0), rows)])
    _banner(f"S={S}: max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= O_TOL[dt] and el <= LSE_TOL


# ------------------------------------------------------------------ edge cases

@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("D", [64, 128])
def test_constant_v_and_causal_row0(dtype, D):
    S = 257
    qb = W.random_bits((1, 2, S, D), dtype, 5)
    kb = W.random_bits((1, 2, S, D), dtype, 6)
    vb = W.round_bits(np.full((1, 2, S, D), 0.8125, np.float32), dtype)
    og, lg = _check_full(qb, kb, vb, dtype, True, D ** -0.5, f"constV D={D} {dtype}")
    assert np.abs(og - 0.8125).max() <= O_TOL[dtype]
    # causal row 0 sees only key 0: O = V[0] (exactly representable), lse = scale*q0.k0
    vb2 = W.random_bits((1, 2, S, D), dtype, 7)
    o, lse = run(qb, kb, vb2, dtype, True, D ** -0.5)
    og2 = o_to_f64(o)
    np.testing.assert_array_equal(og2[:, :, 0], W.decode(vb2[:, :, 0], dtype))


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
def test_identical_keys_closed_form(dtype):
    """All keys equal: O_i = mean of visible V rows, lse_i = scale*q_i.k + ln(i+1)."""
    S, D = 200, 128
    qb = W.random_bits((1, 1, S, D), dtype, 8)
    k1 = W.random_bits((1, 1, 1, D), dtype, 9)
    kb = np.repeat(k1, S, axis=2)
    vb = W.random_bits((1, 1, S, D), dtype, 10)
    o, lse = run(qb, kb, vb, dtype, True, D ** -0.5)
    v = W.decode(vb[0, 0], dtype)
    mean = np.cumsum(v, axis=0) / np.arange(1, S + 1)[:, None]
    q = W.decode(qb[0, 0], dtype)
    k = W.decode(k1[0, 0, 0], dtype)
    lse_ref = float(np.float32(D ** -0.5)) * (q @ k) + np.log(np.arange(1, S + 1))
    assert np.abs(o_to_f64(o)[0, 0] - mean).max() <= O_TOL[dtype]
    assert np.abs(lse.cpu().numpy()[0, 0] - lse_ref).max() <= LSE_TOL


def test_key_shift_moves_lse_only():
    """K += w shifts row i's logits by scale*q_i.w: O unchanged, lse shifted."""
    S, D, dt = 384, 64, W.F16
    q = W.decode(W.random_bits((1, 1, S, D), dt, 11), dt)
    # keys on a 1/64 grid within [-6, 6]: k and k + w are both exact in fp16
    k = np.clip(np.round(W.decode(W.random_bits((1, 1, S, D), dt, 12), dt) * 64) / 64, -6, 6)
    vb = W.random_bits((1, 1, S, D), dt, 13)
    w = np.zeros(D)
    w[:4] = 2.0  # exactly representable shift: k + w stays exact in fp16 here
    kb1 = W.round_bits(k.astype(np.float32), dt)
    kb2 = W.round_bits((k + w).astype(np.float32), dt)
    assert np.array_equal(W.decode(kb2, dt) - W.decode(kb1, dt), np.broadcast_to(w, k.shape))
    qb = W.round_bits(q.astype(np.float32), dt)
    o1, l1 = run(qb, kb1, vb, dt, False, 0.125)
    o2, l2 = run(qb, kb2, vb, dt, False, 0.125)
    assert np.abs(o_to_f64(o1) - o_to_f64(o2)).max() <= O_TOL[dt]
    shift = 0.125 * (q[0, 0] @ w)
    assert np.abs((l2.cpu().numpy() - l1.cpu().numpy())[0, 0] - shift).max() <= 2 * LSE_TOL


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
def test_large_logits_do_not_overflow(dtype):
    """Logits of several hundred: the lagging base keeps every p in (0, 256]."""
    S, D = 256, 64
    qb = W.random_bits((1, 2, S, D), dtype, 14, std=6.0)
    kb = W.random_bits((1, 2, S, D), dtype, 15, std=6.0)
    vb = W.random_bits((1, 2, S, D), dtype, 16)
    _check_full(qb, kb, vb, dtype, False, 0.125, f"large logits {dtype}")


# -------------------------------------------------------- lazy vs eager rescale

def _diag(qb, kb, vb, dtype, causal, scale, thr, variant=0):
    q, k, v = (to_dev(x, dtype) for x in (qb, kb, vb))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=device())
    ev = torch.zeros(1, dtype=torch.int64, device=device())
    B, H, S, D = q.shape
    diag.fa_fwd_diag(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                   B, H, S, D, causal, scale, torch.cuda.current_stream().cuda_stream,
                   W.DTYPE_CODE[dtype], thr, variant, ev.data_ptr())
    torch.cuda.synchronize()
    return o_to_f64(o), lse.cpu().numpy().astype(np.float64), int(ev.item())


@pytest.mark.parametrize("name", ["long", "bat"])
def test_persistent_equals_pingpong_full_size(name):
    """The persistent form runs the ping-pong kernel's per-item code with the
    work items in another order, so at the full workload sizes its output, and
    its count of rescale events, are the ping-pong kernel's bit for bit."""
    w = W.WORKLOADS[name]
    _banner(f"persistent vs ping-pong, {name}: B={w.B} H={w.H} S={w.S} D={w.D}")
    qb, kb, vb = W.make_inputs(w)
    o2, l2, e2 = _diag(qb, kb, vb, w.dtype, w.causal, w.scale, 8, diag.VARIANT_PING_PONG)
    o5, l5, e5 = _diag(qb, kb, vb, w.dtype, w.causal, w.scale, 8, diag.VARIANT_PERSISTENT)
    assert np.array_equal(o2, o5) and np.array_equal(l2, l5)
    assert e5 == e2, (e5, e2)


@pytest.mark.parametrize("kernel", sorted(VARIANTS))
@pytest.mark.parametrize("D", [64, 128])
def test_lagging_and_eager_rescale_both_match(D, kernel):
    """Threshold 8 (production) and 0 (eager) both meet tolerance on a steep
    key ramp; the lag cuts rescale events; event counts track the float64
    model of the same algorithm with the same KV tile size. (The key-split
    kernel runs four passes over interleaved subsets of the tiles, which the
    single-pass model does not describe: its counts are not compared.)"""
    _skip_absent(kernel, D)
    dt = W.BF16
    w = W.Workload("steep", 1, 2, 2048, D, dt, True, 21, ramp=0.05)
    qb, kb, vb = W.make_inputs(w)
    variant = VARIANTS[kernel]
    res = {thr: _diag(qb, kb, vb, dt, True, w.scale, thr, variant) for thr in (8, 0)}
    plan = [((0, h), sample_rows(w.S, 128, seed=h)) for h in range(w.H)]
    for thr, (og, lg, ev) in res.items():
        eo, el = compare_rows(qb, kb, vb, dt, True, w.scale, og, lg, plan)
        _banner(f"D={D} threshold={thr}: events={ev} max|dO|={eo:.3e} max|dlse|={el:.3e}")
        assert eo <= O_TOL[dt] and el <= LSE_TOL
    lazy, eager = res[8][2], res[0][2]
    assert 0 < lazy < eager
    # the production instantiation of the same kernel gives the same bits
    # (same arithmetic, counter aside)
    o, lse = run(qb, kb, vb, dt, True, w.scale, variant=None)
    if kernel == _auto_kernel(D, w.B, w.H, w.S, True):
        np.testing.assert_array_equal(o_to_f64(o), res[8][0])
    if kernel == "sp":
        return
    # the float64 model of the algorithm, same KV tile size
    # KV tile of the forced kernel: the eight-wave kernel's from the tile
    # query on a grid large enough for fa_fwd to pick it
    bn = 64 if kernel in ("k4", "o4") else fa.fa_fwd_tile(D, 1, 256, 1024, True)[1]
    model = {8: 0, 0: 0}
    for h in range(w.H):
        q, k, v = (W.decode(x[0, h], dt) for x in (qb, kb, vb))
        for thr in (8, 0):
            model[thr] += int(oracle.online_softmax_attention(
                q, k, v, True, w.scale, block_n=bn, threshold_log2=thr)["rescales"].sum())
    _banner(f"D={D} model events: lazy={model[8]} eager={model[0]}")
    for thr in (8, 0):
        gpu = res[thr][2]
        assert abs(gpu - model[thr]) <= max(4, 0.02 * model[thr]), (thr, gpu, model[thr])


@pytest.mark.parametrize("h", [0, 3])
def test_ramp_workload_fires_the_lagging_rescale(h):
    """The rescale-stress workload (B=1, H=8, S=16384, D=128, bf16, causal,
    key ramp) exists to exercise the lagging base. On two of its heads the
    production kernel at threshold 8 must rebase (events > 0) as often as the
    float64 model of the same algorithm with the same KV tile predicts, and
    still match the oracle."""
    w = W.WORKLOADS["ramp"]
    _banner(f"ramp head {h}: S={w.S} D={w.D}, threshold 8, ping-pong kernel")
    qb, kb, vb = W.make_inputs(w)
    q1, k1, v1 = (np.ascontiguousarray(x[:, h:h + 1]) for x in (qb, kb, vb))
    og, lg, ev = _diag(q1, k1, v1, w.dtype, True, w.scale, 8, diag.VARIANT_PING_PONG)
    bn = fa.fa_fwd_tile(w.D, 1, 256, 1024, True)[1]  # the ping-pong kernel's KV tile
    q, k, v = (W.decode(x[0, h], w.dtype) for x in (qb, kb, vb))
    model = oracle.online_softmax_attention(q, k, v, True, float(np.float32(w.scale)),
                                            block_n=bn, threshold_log2=8)
    expected = int(model["rescales"].sum())
    _banner(f"ramp head {h}: GPU events={ev} model={expected}")
    assert expected > 0 and ev > 0
    assert abs(ev - expected) <= max(4, 0.02 * expected), (ev, expected)
    eo, el = compare_rows(q1, k1, v1, w.dtype, True, w.scale, og, lg,
                          [((0, 0), sample_rows(w.S, 64, seed=h))])
    _banner(f"ramp head {h}: max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= O_TOL[w.dtype] and el <= LSE_TOL


# ---------------------------------------------------- hygiene of the launch

def test_deterministic():
    shape, dt = (1, 4, 2048, 128), W.BF16
    qb, kb, vb = (W.random_bits(shape, dt, 30 + i) for i in range(3))
    o1, l1 = run(qb, kb, vb, dt, True, 128 ** -0.5)
    o2, l2 = run(qb, kb, vb, dt, True, 128 ** -0.5)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("kernel", sorted(VARIANTS))
@pytest.mark.parametrize("D", [64, 128])
def test_no_writes_outside_outputs(D, kernel):
    """Outputs embedded in guard bands: the kernel writes only O and lse."""
    _skip_absent(kernel, D)
    B, H, S, dt = 1, 3, 200, W.F16
    qb, kb, vb = (W.random_bits((B, H, S, D), dt, 40 + i) for i in range(3))
    q, k, v = (to_dev(x, dt) for x in (qb, kb, vb))
    n, nl, g = B * H * S * D, B * H * S, 4096
    obuf = torch.full((n + 2 * g,), 7.0, dtype=torch.float16, device=device())
    lbuf = torch.full((nl + 2 * g,), -3.0, dtype=torch.float32, device=device())
    o = obuf[g:g + n]
    lse = lbuf[g:g + nl]
    ev = torch.zeros(1, dtype=torch.int64, device=device())
    diag.fa_fwd_diag(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
                   S, D, 1, D ** -0.5, torch.cuda.current_stream().cuda_stream, fa.FA_F16, 8,
                   VARIANTS[kernel], ev.data_ptr())
    torch.cuda.synchronize()
    assert torch.all(obuf[:g] == 7.0) and torch.all(obuf[g + n:] == 7.0)
    assert torch.all(lbuf[:g] == -3.0) and torch.all(lbuf[g + nl:] == -3.0)
    assert torch.all(torch.isfinite(o)) and torch.all(torch.isfinite(lse))


def test_side_stream_and_typed_wrappers():
    shape, dt = (2, 2, 320, 64), W.BF16
    qb, kb, vb = (W.random_bits(shape, dt, 50 + i) for i in range(3))
    ref_o, ref_l = run(qb, kb, vb, dt, True, 0.125)
    s = torch.cuda.Stream()  # default priority
    with torch.cuda.stream(s):
        o, l = run(qb, kb, vb, dt, True, 0.125, stream=s)
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
    q, k, v = (to_dev(x, dt) for x in (qb, kb, vb))
    o2 = torch.empty_like(q)
    l2 = torch.empty_like(ref_l)
    fa.fa_fwd_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                   *shape, 1, 0.125, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(o2, ref_o) and torch.equal(l2, ref_l)


def test_concurrent_host_threads():
    """The library keeps no mutable state: two host threads calling it at once,
    each on its own stream with its own shapes, get exactly the results of
    single-threaded calls."""
    import threading
    cases = [((1, 4, 700, 128), W.BF16, True, 70), ((2, 3, 513, 64), W.F16, False, 80)]
    refs, inputs = [], []
    for shape, dt, causal, seed in cases:
        bits = tuple(W.random_bits(shape, dt, seed + i) for i in range(3))
        inputs.append(tuple(to_dev(x, dt) for x in bits))
        refs.append(run(*bits, dt, causal, shape[3] ** -0.5))
    torch.cuda.synchronize()  # the threads' streams do not wait for these copies
    errors = []

    def worker(n):
        (q, k, v), (_, _, causal, _) = inputs[n], cases[n]
        s = torch.cuda.Stream()  # default priority
        try:
            for _ in range(25):
                with torch.cuda.stream(s):
                    o, l = fa.attention(q, k, v, causal, stream=s)
                s.synchronize()
                if not (torch.equal(o, refs[n][0]) and torch.equal(l, refs[n][1])):
                    errors.append(f"thread {n}: result differs")
                    return
        except Exception as e:  # reported below, in the main thread
            errors.append(f"thread {n}: {e!r}")

    threads = [threading.Thread(target=worker, args=(n,)) for n in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors


def test_empty_inputs_launch_nothing():
    z = torch.empty((0,), dtype=torch.float16, device=device())
    assert fa.fa_fwd(z.data_ptr(), z.data_ptr(), z.data_ptr(), z.data_ptr(), 0, 1, 4, 0, 64, 1,
                     0.125, torch.cuda.current_stream().cuda_stream, fa.FA_F16) == 0
    torch.cuda.synchronize()
