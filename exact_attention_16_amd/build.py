"""Build the gfx950 HIP libraries in-tree:

* exact_attention_16_amd/libfa_fwd.so -- the product library (include/fa_fwd.h);
* exact_attention_16_amd/libfa_fwd_diag.so -- the diagnostic library the tests
  load beside it (include/fa_fwd_diag.h: the same kernels with a
  rescale-event counter, both lag thresholds, and a forced kernel choice);
* exact_attention_16_amd/libfa_probe.so -- the issue-rate probes
  (include/fa_probe.h), run by exact_attention_16_amd.probe.

Usage: python -m exact_attention_16_amd.build [--verbose] [--save-temps DIR]

Compiles all three (in parallel) every time it is called. The code objects target
gfx950 only.
Packed fp32 VALU instructions are disabled for the device code
(-packed-fp32-ops); the host pass warns that it does not know the feature,
which is harmless.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", f) for f in ("fa_fwd.hip", "fa_fwd_fp8.hip")]
OUT = os.path.join(HERE, "libfa_fwd.so")
DIAG_SRCS = [os.path.join(HERE, "csrc", "fa_fwd_diag.hip")]
DIAG_OUT = os.path.join(HERE, "libfa_fwd_diag.so")
PROBE_SRCS = [os.path.join(HERE, "csrc", "fa_probe.hip")]
PROBE_OUT = os.path.join(HERE, "libfa_probe.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA results in arch VGPRs: the softmax reads S with VALU ops
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-I", os.path.join(ROOT, "include"),
        "-Wno-unused-command-line-argument",
    ]


def _command(srcs, out, save_temps):
    # the resource-usage remarks are always on: scratch_use() checks them
    cmd = [hipcc(), *compile_flags(), *srcs, "-o", out + ".tmp",
           "-Rpass-analysis=kernel-resource-usage"]
    if save_temps:
        cmd += ["-save-temps=obj"]
        cmd[cmd.index("-o") + 1] = os.path.abspath(out + ".tmp")
    return cmd


def scratch_use(remarks: str) -> list[tuple[str, int]]:
    """Kernels whose resource-usage remarks report scratch memory (register
    spills), with the bytes per lane. No kernel here may spill: besides the
    cost, the ping-pong kernel counts its vector-memory instructions exactly
    in its waits (a constant count of DMA issues left in flight), and spill
    loads and stores would make those waits too short."""
    out, name = [], None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:", 1)[1].split()[0]
        elif "ScratchSize [bytes/lane]:" in line and name:
            n = int(line.split("ScratchSize [bytes/lane]:", 1)[1].split()[0])
            if n > 0:
                out.append((name, n))
    return out


def build(verbose: bool = False, save_temps: str | None = None, resource_usage: bool = False,
          diag: bool = True) -> str:
    """Compile the product library (and the diagnostic and probe libraries
    unless diag=False); returns the product library's path."""
    jobs = [(SRCS, OUT)] + ([(DIAG_SRCS, DIAG_OUT), (PROBE_SRCS, PROBE_OUT)] if diag else [])
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
    procs = []
    for srcs, out in jobs:
        cmd = _command(srcs, out, save_temps)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((out, subprocess.Popen(cmd, cwd=save_temps or None, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
    failed = []
    for out, p in procs:
        text, _ = p.communicate()
        # the host pass does not know the device-only target feature
        text = "\n".join(l for l in (text or "").splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(f"{os.path.basename(out)}: hipcc failed ({p.returncode}):\n{text}")
            continue
        if verbose or resource_usage:
            print(text, flush=True)
        spills = scratch_use(text)
        if spills:
            os.remove(out + ".tmp")
            failed.append(f"{os.path.basename(out)}: kernels use scratch memory: "
                          + ", ".join(f"{n} ({b} bytes/lane)" for n, b in spills))
            continue
        os.replace(out + ".tmp", out)
    if failed:
        raise RuntimeError("\n".join(failed))
    return OUT


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    ap.add_argument("--save-temps", default=None)
    ap.add_argument("--no-diag", action="store_true", help="build the product library only (no diagnostic or probe library)")
    a = ap.parse_args(argv)
    p = build(a.verbose, a.save_temps, a.resource_usage, diag=not a.no_diag)
    print(p)
    return 0


if __name__ == "__main__":
    sys.exit(main())
