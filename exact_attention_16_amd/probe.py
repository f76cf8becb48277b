"""Issue-rate probes of one gfx950 compute unit (libfa_probe.so, declared in
include/fa_probe.h): how often a SIMD issues v_fma_f32, v_exp_f32 and
v_mfma_f32_32x32x16_bf16, alone and side by side, with 1 to 4 waves per
SIMD. These are the rates the attention kernels' schedules are built on.

Usage: python -m exact_attention_16_amd.probe [--out FILE]   (needs the GPU)

Prints a markdown report (and writes it to FILE). Every figure is in shader
clock cycles (s_memtime), so it does not depend on the clock the GPU runs
at. Argument marshalling over ctypes; torch supplies the device buffer.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import statistics
import sys

from exact_attention_16_amd import _lib

PROBE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_probe.so")

NONE, FMA, EXP, MFMA, MIX, MFMA_DEP = 0, 1, 2, 3, 4, 5
# instructions per block of each stream (MIX: exponentials per block)
PER_BLOCK = {FMA: 32, EXP: 32, MFMA: 16, MIX: 32, MFMA_DEP: 16}
NAMES = {FMA: "v_fma_f32", EXP: "v_exp_f32", MFMA: "v_mfma_f32_32x32x16_bf16", MIX: "mix",
         MFMA_DEP: "v_mfma_f32_32x32x16_bf16, dependent"}

SIGNATURES = {
    "fa_probe_run": (ctypes.c_int, [ctypes.c_int] * 6 + [ctypes.c_void_p, ctypes.c_void_p]),
}

_probe = None


def load_probe() -> ctypes.CDLL:
    global _probe
    if _probe is None:
        if not os.path.exists(PROBE_PATH):
            raise RuntimeError(f"{PROBE_PATH} is not built; run `python -m exact_attention_16_amd.build`")
        lib = ctypes.CDLL(PROBE_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _probe = lib
    return _probe


def fa_probe_run(a, iters_a, b, iters_b, waves_per_simd, mix, out_ptr, stream, check=True):
    st = load_probe().fa_probe_run(a, iters_a, b, iters_b, waves_per_simd, mix, out_ptr, stream)
    if check and st != 0:
        raise _lib.FaError(st, "fa_probe_run")
    return st


def run(a, iters_a, b=NONE, iters_b=0, waves_per_simd=1, mix=0, repeats=3):
    """One probe launch per repeat; returns, per wave, (median cycles, SIMD,
    CU). Checks that waves 0-3 ran on four different SIMDs and wave w on the
    SIMD of wave w mod 4, all on one CU."""
    import torch
    n = 4 * waves_per_simd
    out = torch.zeros(3 * n, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    cyc = [[] for _ in range(n)]
    where = None
    fa_probe_run(a, iters_a, b, iters_b, waves_per_simd, mix, out.data_ptr(), stream)  # warm-up
    for _ in range(repeats):
        out.zero_()
        fa_probe_run(a, iters_a, b, iters_b, waves_per_simd, mix, out.data_ptr(), stream)
        r = out.view(n, 3).cpu().tolist()
        for w in range(n):
            cyc[w].append(r[w][0])
        where = [(r[w][1], r[w][2]) for w in range(n)]
    if len({s for s, _ in where[:4]}) != 4:
        raise RuntimeError(f"waves 0-3 ran on SIMDs {[s for s, _ in where[:4]]}: the probes "
                           "assume four different SIMDs")
    for w, (simd, cu) in enumerate(where):
        if simd != where[w % 4][0] or cu != where[0][1]:
            raise RuntimeError(f"wave {w} ran on SIMD {simd} of CU {cu}: the probes assume "
                               f"SIMD {where[w % 4][0]} of CU {where[0][1]}")
    return [(statistics.median(c), s, cu) for c, (s, cu) in zip(cyc, where)]


def _slot_cycles(res, slot):
    """Median over the four SIMDs of slot `slot`'s wave cycles."""
    return statistics.median(res[4 * slot + s][0] for s in range(4))


def measure() -> dict:
    """The figures of the report, as a dict of named values (cycles)."""
    m = {}
    it = {FMA: 1000, EXP: 250, MFMA: 125}
    for kind in (FMA, EXP, MFMA):
        n_inst = PER_BLOCK[kind] * it[kind]
        for wps in (1, 2, 3, 4):
            res = run(kind, it[kind], kind, it[kind], wps)
            longest = max(c for c, _, _ in res)
            m[(NAMES[kind], wps, "per_wave")] = _slot_cycles(res, 0) / n_inst
            m[(NAMES[kind], wps, "per_simd")] = longest / (wps * n_inst)
    # latency: one accumulator, each MFMA the addend of the next
    res = run(MFMA_DEP, 125, NONE, 0, 1)
    m[("dep",)] = _slot_cycles(res, 0) / (PER_BLOCK[MFMA_DEP] * 125)
    # one wave: exponentials, each followed by R independent FMAs
    for wps in (1, 2):
        for r in (0, 1, 2, 3, 4, 6, 8):
            res = run(MIX, 250, MIX, 250, wps, r)
            m[("mix", wps, r)] = _slot_cycles(res, 0) / (PER_BLOCK[MIX] * 250)
    # side by side: slot 0 of each SIMD runs stream A, the other slots stream B
    pairs = [(MFMA, EXP), (MFMA, FMA), (EXP, FMA)]
    for a, b in pairs:
        for wps in (2, 4):
            ia, ib = it[a], it[b]
            alone_a = _slot_cycles(run(a, ia, NONE, 0, wps), 0)
            alone_b = _slot_cycles(run(NONE, 0, b, ib, wps), 1)
            both = run(a, ia, b, ib, wps)
            m[(NAMES[a], NAMES[b], wps)] = (alone_a, alone_b, _slot_cycles(both, 0),
                                            _slot_cycles(both, 1))
    return m


def report(m: dict) -> str:
    L = ["# Issue rates of one gfx950 SIMD (shader clock cycles)", "",
         "Command: `python -m exact_attention_16_amd.probe --out profiles/issue_rates.md` "
         "(one work-group on one CU; waves 0-3 on four different SIMDs and wave w on the SIMD of wave w mod 4, checked from HW_ID; median of 3).", "",
         "## One stream on every wave", "",
         "Eight independent chains per wave (four accumulators for the MFMA), so a chain's "
         "latency does not set the rate. `per wave`: cycles between a wave's instructions; "
         "`per SIMD`: cycles per instruction issued by all the SIMD's waves together.", "",
         "| instruction | waves per SIMD | cycles per instruction, per wave | per SIMD |",
         "|---|---|---|---|"]
    for kind in (FMA, EXP, MFMA):
        for wps in (1, 2, 3, 4):
            L.append(f"| {NAMES[kind]} | {wps} | {m[(NAMES[kind], wps, 'per_wave')]:.2f} | "
                     f"{m[(NAMES[kind], wps, 'per_simd')]:.2f} |")
    L += ["", f"Dependent v_mfma_f32_32x32x16_bf16 (one accumulator, each the addend of the next), "
          f"one wave per SIMD: {m[('dep',)]:.2f} cycles per instruction.", "",
          "## Exponentials with independent FMAs in one wave", "",
          "Each v_exp_f32 followed by R v_fma_f32 of other chains; cycles per (exp + R FMAs) "
          "group, for the wave in slot 0 (with 2 waves per SIMD both run the same stream).", "",
          "| R | 1 wave per SIMD | 2 waves per SIMD |", "|---|---|---|"]
    for r in (0, 1, 2, 3, 4, 6, 8):
        L.append(f"| {r} | {m[('mix', 1, r)]:.2f} | {m[('mix', 2, r)]:.2f} |")
    L += ["", "## Two streams side by side", "",
          "Slot 0 of each SIMD runs stream A, the other waves of the SIMD stream B. Cycles of "
          "each stream's waves alone (the other slots idle) and together.", "",
          "| A | B | waves per SIMD | A alone | B alone | A beside B | B beside A |",
          "|---|---|---|---|---|---|---|"]
    for a, b in [(MFMA, EXP), (MFMA, FMA), (EXP, FMA)]:
        for wps in (2, 4):
            aa, ba, ab, bb = m[(NAMES[a], NAMES[b], wps)]
            L.append(f"| {NAMES[a]} | {NAMES[b]} | {wps} | {aa:,.0f} | {ba:,.0f} | {ab:,.0f} | "
                     f"{bb:,.0f} |")
    return "\n".join(L) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None)
    a = ap.parse_args(argv)
    import torch
    if not torch.cuda.is_available():
        print("the probes need a GPU", file=sys.stderr)
        return 2
    text = report(measure())
    print(text, flush=True)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
