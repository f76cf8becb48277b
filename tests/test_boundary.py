"""The C-ABI boundary without a GPU: exported symbols, argument validation
(which runs on the host before any HIP call) and the kernel's index math."""
import os
import re
import shutil
import subprocess

import pytest

import diag
import exact_attention_16_amd as fa
from exact_attention_16_amd import _lib, probe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_fwd.h")
DIAG_HEADER = os.path.join(ROOT, "include", "fa_fwd_diag.h")
PROBE_HEADER = os.path.join(ROOT, "include", "fa_probe.h")

OK, NULL, DIM, UNSUP, ALIGN, SCALE, ALIAS, HIP, ARG, LAYOUT = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9


def _declared(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M))


def _exported(path):
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("no nm")
    out = subprocess.run([nm, "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    return set(re.findall(r" T (fa_\w+)$", out, flags=re.M))


def test_header_declares_the_entry_points():
    assert _declared() == {"fa_fwd", "fa_fwd_f16", "fa_fwd_bf16", "fa_fwd_strided",
                           "fa_fwd_varlen", "fa_fwd_kt", "fa_fwd_fp8", "fa_fwd_tile",
                           "fa_strerror", "fa_version"}
    assert _declared(DIAG_HEADER) == {"fa_fwd_diag"}
    assert _declared(PROBE_HEADER) == {"fa_probe_run"}


def test_library_exports_every_declared_symbol():
    """The product library exports exactly the product header's entry points
    (no diagnostic hook); the diagnostic library exactly its own."""
    lib = fa.load()
    for name in _declared():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, name
    assert _exported(fa.LIB_PATH) == _declared()
    dlib = diag.load_diag()
    for name in _declared(DIAG_HEADER):
        assert hasattr(dlib, name), name
        assert name in diag.SIGNATURES, name
    assert _exported(diag.DIAG_PATH) == _declared(DIAG_HEADER)
    plib = probe.load_probe()
    for name in _declared(PROBE_HEADER):
        assert hasattr(plib, name), name
        assert name in probe.SIGNATURES, name
    assert _exported(probe.PROBE_PATH) == _declared(PROBE_HEADER)


def _stubs(path):
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("no nm")
    out = subprocess.run([nm, "-D", path], capture_output=True, text=True, check=True).stdout
    return [l for l in out.splitlines() if "device_stub" in l]


def test_kernel_launch_stubs_are_defined():
    """Every kernel instantiation the launchers reference has a host stub."""
    stubs = _stubs(fa.LIB_PATH)
    # product: 2 kernels (ping-pong, four-wave) x 2 dtypes x 2 head dims x 2
    # masks, the key-split kernel x 2 dtypes x 2 masks (D = 64), the
    # four-waves-per-SIMD kernel x 2 dtypes (D = 64, no mask), the
    # transposed-K kernel x 2 x 2 x 2, the 8-bit kernel x 2 x 2
    assert len(stubs) == 34
    assert not [l for l in stubs if l.split()[-2] == "U"], "undefined kernel stubs"
    assert not [l for l in stubs if "ELb1EEEv" in l and "fa_fwd_pp_kt" not in l
                and "fa_fwd_il8" not in l], "instrumented kernels in the product library"
    dstubs = _stubs(diag.DIAG_PATH)
    # diagnostic: 3 kernels (four-wave, ping-pong, persistent) x 2 dtypes x 2
    # head dims x 2 masks x 2 lag thresholds, the key-split and the
    # four-waves-per-SIMD kernels x 2 dtypes x 2 masks x 2 thresholds (D = 64)
    assert len(dstubs) == 64
    assert not [l for l in dstubs if l.split()[-2] == "U"], "undefined kernel stubs"


def test_version_and_strerror():
    assert fa.fa_version() == 500
    for st in (OK, NULL, DIM, UNSUP, ALIGN, SCALE, ALIAS, HIP, ARG, LAYOUT):
        assert fa.fa_strerror(st) and fa.fa_strerror(st) != "unknown status"
    assert fa.fa_strerror(12345) == "unknown status"


def test_tile_query():
    # at D = 64 without the causal mask the four-waves-per-SIMD kernel (256
    # rows, 64-key tiles) where the eight-wave kernel would run; eight-wave
    # kernel once B*H*ceil(S/256) >= 256 work-groups; else the four-wave
    # kernel once B*H*ceil(S/128) >= 256, at D = 128 or for S < 256; else the
    # key-split kernel (64 rows, four groups of two waves)
    assert fa.fa_fwd_tile(128, 2, 16, 8192, True) == (256, 96, 512, 2 * 16 * 32)
    assert fa.fa_fwd_tile(128, 2, 16, 8192, False) == (256, 96, 512, 2 * 16 * 32)
    assert fa.fa_fwd_tile(64, 10, 64, 1024) == (256, 64, 512, 640 * 4)
    assert fa.fa_fwd_tile(64, 10, 64, 1024, True) == (256, 128, 512, 640 * 4)
    assert fa.fa_fwd_tile(64, 1, 64, 1024, False) == (256, 64, 512, 256)
    assert fa.fa_fwd_tile(64, 1, 63, 1024, False) == (128, 64, 256, 63 * 8)
    assert fa.fa_fwd_tile(64, 1, 16, 1024) == (64, 64, 512, 16 * 16)
    assert fa.fa_fwd_tile(64, 1, 32, 1024) == (128, 64, 256, 32 * 8)
    assert fa.fa_fwd_tile(128, 1, 64, 1024) == (256, 96, 512, 256)
    assert fa.fa_fwd_tile(128, 1, 63, 1024) == (128, 64, 256, 63 * 8)
    assert fa.fa_fwd_tile(128, 1, 16, 1024) == (128, 64, 256, 16 * 8)
    assert fa.fa_fwd_tile(64, 1, 1, 129) == (128, 64, 256, 2)
    assert fa.fa_fwd_tile(64, 1, 1, 256) == (64, 64, 512, 4)
    with pytest.raises(fa.FaError):
        fa.fa_fwd_tile(96)
    with pytest.raises(fa.FaError, match="FA_ERR_ARG"):
        fa.fa_fwd_tile(64, 1, 1, 64, 2)


# fake, 16-byte aligned, non-overlapping device addresses: validation never
# dereferences them and rejects every case below before any HIP call
N = 1 << 30
Q, K, V, O, L = (0x10000000000 + i * 4 * N for i in range(5))
GOOD = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, S=100, D=64, causal=1, scale=0.125,
            stream=None, dtype=0)


def _call(**kw):
    a = dict(GOOD, **kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["S"], a["D"],
                     a["causal"], a["scale"], a["stream"], a["dtype"], check=False)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), NULL), (dict(k=0), NULL), (dict(v=0), NULL), (dict(o=0), NULL),
    (dict(lse=0), NULL),
    (dict(B=-1), DIM), (dict(H=-2), DIM), (dict(S=-5), DIM), (dict(S=(1 << 30) + 1), DIM),
    (dict(B=1 << 20, H=1 << 10, S=1 << 12), DIM),
    (dict(D=96), UNSUP), (dict(D=0), UNSUP), (dict(D=256), UNSUP), (dict(dtype=2), UNSUP),
    (dict(dtype=-1), UNSUP),
    (dict(q=Q + 8), ALIGN), (dict(o=O + 2), ALIGN), (dict(lse=L + 4), ALIGN),
    (dict(scale=0.0), SCALE), (dict(scale=-0.1), SCALE), (dict(scale=float("nan")), SCALE),
    (dict(scale=float("inf")), SCALE),
    (dict(o=Q), ALIAS), (dict(o=K + 1024), ALIAS), (dict(lse=V + 64), ALIAS),
    (dict(lse=O + 16), ALIAS), (dict(o=V - 16), ALIAS),
    (dict(causal=2), ARG), (dict(causal=-1), ARG),
])
def test_validation_rejects(kw, expect):
    assert _call(**kw) == expect


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(S=0),
                                dict(S=0, q=0, k=0, v=0, o=0, lse=0)])
def test_empty_problem_is_a_noop(kw):
    assert _call(**kw) == OK


def test_typed_wrappers_validate_the_same_way():
    a = GOOD
    assert fa.fa_fwd_f16(a["q"], a["k"], a["v"], 0, a["lse"], 1, 1, 8, 64, 0, 0.1, None,
                         check=False) == NULL
    assert fa.fa_fwd_bf16(a["q"], a["k"], a["v"], a["o"], a["lse"], 1, 1, 8, 64, 0, -1.0, None,
                          check=False) == SCALE
    assert fa.fa_fwd_bf16(a["q"], a["k"], a["v"], a["o"], a["lse"], 1, 1, 0, 64, 0, 0.1, None,
                          check=False) == OK


def test_diag_validation():
    a = GOOD
    args = (a["q"], a["k"], a["v"], a["o"], a["lse"], 1, 1, 8, 64, 0, 0.1, None, 0)
    ev = 0x20000000000
    assert diag.fa_fwd_diag(*args, 3, 0, ev, check=False) == ARG
    for retired in (3, 4, 6, -1):
        assert diag.fa_fwd_diag(*args, 8, retired, ev, check=False) == ARG
    # the key-split kernel exists at D = 64 only
    args128 = (a["q"], a["k"], a["v"], a["o"], a["lse"], 1, 1, 4, 128, 0, 0.1, None, 0)
    assert diag.fa_fwd_diag(*args128, 8, diag.VARIANT_SPLIT, ev, check=False) == ARG
    assert diag.fa_fwd_diag(*args128, 8, diag.VARIANT_OCC4, ev, check=False) == ARG
    for bad in (6, 9):
        assert diag.fa_fwd_diag(*args, 8, bad, ev, check=False) == ARG
    assert diag.fa_fwd_diag(*args, 8, 0, 0, check=False) == NULL
    assert diag.fa_fwd_diag(*args, 0, 2, ev + 4, check=False) == ALIGN
    # the product checks run first
    bad = (a["q"], a["k"], a["v"], a["q"], a["lse"], 1, 1, 8, 64, 0, 0.1, None, 0)
    assert diag.fa_fwd_diag(*bad, 8, 0, ev, check=False) == ALIAS
    e = (a["q"], a["k"], a["v"], a["o"], a["lse"], 1, 1, 0, 64, 0, 0.1, None, 0)
    for variant in (0, 1, 2, 5):
        assert diag.fa_fwd_diag(*e, 8, variant, ev, check=False) == OK


@pytest.mark.parametrize("args,expect", [
    ((probe.NONE, 1, probe.NONE, 1, 1, 0), ARG),      # no stream at all
    ((6, 1, probe.NONE, 0, 1, 0), ARG),               # unknown stream
    ((probe.FMA, 1, -1, 1, 1, 0), ARG),
    ((probe.FMA, 0, probe.NONE, 0, 1, 0), ARG),       # iters out of range
    ((probe.FMA, (1 << 20) + 1, probe.NONE, 0, 1, 0), ARG),
    ((probe.FMA, 1, probe.EXP, 0, 2, 0), ARG),
    ((probe.FMA, 1, probe.NONE, 0, 0, 0), ARG),       # waves per SIMD out of range
    ((probe.FMA, 1, probe.NONE, 0, 5, 0), ARG),
    ((probe.MIX, 1, probe.NONE, 0, 1, 9), ARG),       # mix out of range
    ((probe.MIX, 1, probe.NONE, 0, 1, -1), ARG),
])
def test_probe_validation(args, expect):
    assert probe.fa_probe_run(*args, 0x20000000000, None, check=False) == expect


def test_probe_null_and_alignment():
    assert probe.fa_probe_run(probe.FMA, 1, probe.NONE, 0, 1, 0, 0, None, check=False) == NULL
    assert probe.fa_probe_run(probe.FMA, 1, probe.NONE, 0, 1, 0, 0x20000000004, None,
                              check=False) == ALIGN


def test_error_raises_with_name():
    with pytest.raises(fa.FaError, match="FA_ERR_NULL"):
        fa.fa_fwd(0, 0, 0, 0, 0, 1, 1, 8, 64, 0, 0.1, None, 0)


def test_kernel_index_math_on_host(tmp_path):
    """Bounds, exact LDS coverage, operand element mapping, work decomposition
    and LDS bank-conflict degree of every access the kernel makes."""
    gxx = shutil.which("g++") or shutil.which("c++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "layout_check"
    subprocess.run([gxx, "-std=c++17", "-O2", "-o", str(exe),
                    os.path.join(ROOT, "tests", "host", "layout_check.cpp")], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout


# ------------------------------------------------ strided and variable-length
B_, H_, SQ, SK, D_ = 2, 3, 100, 80, 64


def _dense(B, H, Sq, Sk, D):
    """14 strides of contiguous [B,H,S,D] q/k/v/o and [B,H,Sq] lse."""
    q = [H * Sq * D, Sq * D, D]
    k = [H * Sk * D, Sk * D, D]
    return q + k + k + q + [H * Sq, Sq]


def _strided(strides=None, **kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, B=B_, H=H_, Sq=SQ, Sk=SK, D=D_, causal=1, scale=0.125,
             dtype=0)
    a.update(kw)
    st = _dense(B_, H_, SQ, SK, D_) if strides is None else strides
    return fa.fa_fwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Sq"],
                             a["Sk"], a["D"], a["causal"], a["scale"], None, a["dtype"], st,
                             check=False)


def _with(i, x):
    st = _dense(B_, H_, SQ, SK, D_)
    st[i] = x
    return st


@pytest.mark.parametrize("strides,kw,expect", [
    (None, dict(q=0), NULL), (None, dict(lse=0), NULL),
    (None, dict(Sq=-1), DIM), (None, dict(Sk=-1), DIM), (None, dict(D=80), UNSUP),
    (None, dict(scale=0.0), SCALE), (None, dict(causal=3), ARG),
    (_with(2, -64), {}, LAYOUT),            # negative row stride
    (_with(5, 32), {}, LAYOUT),             # k rows shorter than D
    (_with(11, 8), {}, LAYOUT),             # o rows overlap each other
    (_with(10, 64), {}, LAYOUT),            # o heads overlap (head stride one row)
    (_with(13, 1), {}, LAYOUT),             # lse heads overlap
    (_with(2, 68), {}, ALIGN),              # q rows not 16-byte aligned
    (_with(7, 64 * 3 + 4), {}, ALIGN),      # v heads not 16-byte aligned
    (_with(11, 1 << 24), {}, DIM),          # 32-bit offsets within one head
    (_with(1, 1 << 62), {}, DIM),           # q head stride: (H-1)*stride overflows 64 bits
    (_with(0, (1 << 62) + 8), {}, DIM),     # q batch stride likewise
    (_with(10, 1 << 41), {}, DIM),          # above the 2^40 stride cap
    (_with(13, 1 << 62), {}, DIM),          # lse head stride
    (None, dict(o=K + 4096), ALIAS),        # o inside k's span
    (None, dict(lse=O + 64), ALIAS),
])
def test_strided_validation(strides, kw, expect):
    assert _strided(strides, **kw) == expect


def test_strided_needs_strides_and_empty_is_a_noop():
    assert _lib.load().fa_fwd_strided(Q, K, V, O, L, 1, 1, 8, 8, 64, 0, 0.1, None, 0,
                                      None) == NULL
    assert _strided(Sq=0) == OK
    assert _strided(B=0) == OK
    assert _lib.load().fa_fwd_strided(0, 0, 0, 0, 0, 1, 1, 0, 8, 64, 0, 0.1, None, 0, None) == OK


def _varlen_call(cu_q=0x30000000000, cu_k=0x30000001000, total_q=50, total_k=60, strides=None,
                 **kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, B=4, H=2, mq=20, mk=30, D=64, causal=1, scale=0.125,
             dtype=1)
    a.update(kw)
    # packed [total, H, D]: head stride D, row stride H*D; lse [H, total_q]
    st = [64, 128, 64, 128, 64, 128, 64, 128, total_q] if strides is None else strides
    return fa.fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], cu_q, cu_k, a["B"], a["H"],
                            a["mq"], a["mk"], total_q, total_k, a["D"], a["causal"], a["scale"],
                            None, a["dtype"], st, check=False)


# (inputs may overlap themselves: they are read only; only outputs are checked)
@pytest.mark.parametrize("args,expect", [
    (dict(cu_q=0), NULL), (dict(cu_k=0), NULL), (dict(cu_q=0x30000000002), ALIGN),
    (dict(total_q=-1), DIM), (dict(total_k=-1), DIM), (dict(B=-1), DIM),
    (dict(D=32), UNSUP), (dict(scale=-1.0), SCALE), (dict(causal=5), ARG),
    (dict(q=0), NULL),
    (dict(strides=[64, 128, 64, 128, 64, 128, 64, 64, 50]), LAYOUT),   # o rows overlap
    (dict(strides=[64, 128, 64, 128, 64, 128, 64, 128, 10]), LAYOUT),  # lse heads overlap
    (dict(strides=[64, 132, 64, 128, 64, 128, 64, 128, 50]), ALIGN),
    (dict(o=V + 256), ALIAS),
])
def test_varlen_validation(args, expect):
    assert _varlen_call(**args) == expect


@pytest.mark.parametrize("args", [dict(total_q=0), dict(B=0), dict(mq=0),
                                  dict(total_q=0, cu_q=0, cu_k=0, q=0)])
def test_varlen_empty_is_a_noop(args):
    assert _varlen_call(**args) == OK


# ------------------------------------------------ 8-bit inputs
GOOD8 = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, S=100, D=128, causal=1, scale=0.125,
             dq=0.01, dk=0.02, dv=0.5, stream=None)


def _call8(**kw):
    a = dict(GOOD8, **kw)
    return fa.fa_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["S"],
                         a["D"], a["causal"], a["scale"], a["dq"], a["dk"], a["dv"], a["stream"],
                         check=False)


NBYTES = 2 * 3 * 100 * 128  # one 8-bit input tensor of GOOD8


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), NULL), (dict(v=0), NULL), (dict(o=0), NULL), (dict(lse=0), NULL),
    (dict(B=-1), DIM), (dict(S=-1), DIM), (dict(S=1 << 23), DIM),
    (dict(B=1 << 16, H=1 << 16, S=1 << 12), DIM),
    (dict(D=96), UNSUP), (dict(D=256), UNSUP),
    (dict(k=K + 8), ALIGN), (dict(lse=L + 4), ALIGN),
    (dict(scale=0.0), SCALE), (dict(dq=0.0), SCALE), (dict(dk=-1.0), SCALE),
    (dict(dv=float("nan")), SCALE), (dict(dv=float("inf")), SCALE),
    (dict(scale=1e-30, dq=1e-10), SCALE),          # folded multiplier underflows
    (dict(scale=1e30, dq=1e10, dk=1e10), SCALE),   # overflows
    # q, k, v span one byte per element, o two, lse four per row
    (dict(o=Q + NBYTES - 16), ALIAS), (dict(o=V - 2 * NBYTES + 16), ALIAS),
    (dict(lse=O + 2 * NBYTES - 16), ALIAS), (dict(lse=K), ALIAS),
    (dict(causal=2), ARG),
])
def test_fp8_validation_rejects(kw, expect):
    assert _call8(**kw) == expect


def test_fp8_empty_problem_is_a_noop():
    assert _call8(S=0) == OK
    assert _call8(B=0, q=0, k=0, v=0, o=0, lse=0) == OK
    assert _call8(H=0, D=96) == UNSUP  # the head dimension is checked first


# ------------------------------------------------ K given transposed
def _call_kt(**kw):
    a = dict(GOOD, S=104)
    a.update(kw)
    return fa.fa_fwd_kt(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["S"], a["D"],
                        a["causal"], a["scale"], a["stream"], a["dtype"], check=False)


@pytest.mark.parametrize("kw,expect", [
    (dict(k=0), NULL), (dict(lse=0), NULL), (dict(B=-1), DIM), (dict(D=96), UNSUP),
    (dict(dtype=3), UNSUP), (dict(S=100), ALIGN), (dict(S=7), ALIGN), (dict(k=K + 8), ALIGN),
    (dict(scale=0.0), SCALE), (dict(o=K + 64), ALIAS), (dict(lse=O + 32), ALIAS),
    (dict(causal=3), ARG),
])
def test_kt_validation_rejects(kw, expect):
    assert _call_kt(**kw) == expect


def test_kt_empty_problem_is_a_noop():
    assert _call_kt(S=0) == OK
    assert _call_kt(B=0, q=0, k=0, v=0, o=0, lse=0) == OK


# ------------------------------------------------ torch helpers, host side
def test_torch_helpers_reject_host_tensors_before_any_launch():
    import torch
    q = torch.zeros((1, 1, 8, 64), dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.attention(q, q, q, True)
    with pytest.raises(ValueError):
        fa.attention_kt(q, q.transpose(-1, -2).contiguous(), q, True)
    q8 = torch.zeros((1, 1, 8, 128), dtype=torch.uint8)
    with pytest.raises(ValueError):
        fa.attention_fp8(q8, q8, q8, 1.0, 1.0, 1.0, True)
    with pytest.raises(ValueError):
        fa.attention_varlen(q[0, 0][:, None, :], q[0, 0][:, None, :], q[0, 0][:, None, :],
                            torch.zeros(2, dtype=torch.int32), torch.zeros(2, dtype=torch.int32),
                            8, 8, True)


@pytest.mark.parametrize("bad,match", [
    (dict(out_dtype="float32"), "out must be"),       # 4-byte elements into a 2-byte output
    (dict(out_shape=(1, 2, 7, 64)), "out must have shape"),
    (dict(lse_dtype="float16"), "lse must be float32"),  # 4-byte stores into 2-byte lse
    (dict(lse_shape=(1, 2, 4)), "lse must have shape"),
])
def test_torch_helpers_check_out_and_lse_before_any_launch(bad, match):
    """A caller-supplied out or lse of the wrong type or shape would be
    written past its end by the kernel (the C side sees only pointers):
    the helpers refuse it first."""
    import torch
    dt = {"float32": torch.float32, "float16": torch.float16}
    q = torch.zeros((1, 2, 8, 64), dtype=torch.float16)
    out = torch.zeros(bad.get("out_shape", (1, 2, 8, 64)), dtype=dt[bad.get("out_dtype", "float16")])
    lse = torch.zeros(bad.get("lse_shape", (1, 2, 8)), dtype=dt[bad.get("lse_dtype", "float32")])
    with pytest.raises(ValueError, match=match):
        fa.attention(q, q, q, True, out=out, lse=lse)
    with pytest.raises(ValueError, match=match):
        fa.attention(q, q, q, True, out=out, lse=lse, layout="bhsd")
    with pytest.raises(ValueError, match=match):
        fa.attention_kt(q, q.transpose(-1, -2).contiguous(), q, True, out=out, lse=lse)
    # varlen: q [total, H, D], out the same, lse [H, total]
    qv = torch.zeros((8, 2, 64), dtype=torch.float16)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    out_v = torch.zeros(bad.get("out_shape", (8, 2, 64))[-3:] if "out_shape" in bad else (8, 2, 64),
                        dtype=dt[bad.get("out_dtype", "float16")])
    lse_v = torch.zeros((2, 8) if "lse_shape" not in bad else (2, 4),
                        dtype=dt[bad.get("lse_dtype", "float32")])
    if "out_shape" in bad:
        out_v = torch.zeros((7, 2, 64), dtype=torch.float16)
    with pytest.raises(ValueError, match=match):
        fa.attention_varlen(qv, qv, qv, cu, cu, 8, 8, True, out=out_v, lse=lse_v)
    # 8-bit: out must be bf16
    q8 = torch.zeros((1, 2, 8, 64), dtype=torch.uint8)
    out8 = torch.zeros(bad.get("out_shape", (1, 2, 8, 64)),
                       dtype=torch.float32 if "out_dtype" in bad else torch.bfloat16)
    with pytest.raises(ValueError, match=match):
        fa.attention_fp8(q8, q8, q8, 1.0, 1.0, 1.0, True, out=out8, lse=lse)


def test_torch_helpers_check_the_device_of_out():
    """out on another device than q (a host buffer for a device q) is refused.
    Without a GPU, q itself is on the host, so a meta-device out stands in."""
    import torch
    q = torch.zeros((1, 1, 8, 64), dtype=torch.float16)
    out = torch.empty((1, 1, 8, 64), dtype=torch.float16, device="meta")
    with pytest.raises(ValueError, match="out must be on"):
        fa.attention(q, q, q, True, out=out)


def test_binding_fails_loudly_without_the_library(tmp_path, monkeypatch):
    """No library, no fallback: loading raises and names the build step."""
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load()
    with pytest.raises(RuntimeError, match="not built"):
        _lib.fa_version()


def test_product_path_does_not_import_the_oracle():
    """The package and the benchmark's timed path never touch oracle/."""
    pkg = os.path.join(ROOT, "exact_attention_16_amd")
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            text = open(os.path.join(pkg, name)).read()
            assert "oracle" not in text, name
    bench = open(os.path.join(ROOT, "bench.py")).read()
    # the only use: the cpu_baseline leg, imported inside that function
    assert bench.count("import oracle") == 1
    assert "def cpu_baseline" in bench.split("import oracle")[0].rsplit("\n\n\n", 1)[-1]
