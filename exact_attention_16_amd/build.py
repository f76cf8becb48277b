"""Build the gfx950 HIP library in-tree: exact_attention_16_amd/libfa_fwd.so.

Usage: python -m exact_attention_16_amd.build [--verbose] [--save-temps DIR]

Compiles every time it is called. The code object targets gfx950 only.
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


def build(verbose: bool = False, save_temps: str | None = None, resource_usage: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = [hipcc(), *compile_flags(), *SRCS, "-o", tmp]
    if resource_usage:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd += [f"-save-temps={'obj'}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    cwd = save_temps or None
    if save_temps:
        cmd[cmd.index("-o") + 1] = os.path.abspath(tmp)
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    out = (r.stdout or "") + (r.stderr or "")
    # the host pass does not know the device-only target feature
    out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{out}")
    if verbose or resource_usage:
        print(out, flush=True)
    os.replace(tmp, OUT)
    return OUT


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    ap.add_argument("--save-temps", default=None)
    a = ap.parse_args(argv)
    p = build(a.verbose, a.save_temps, a.resource_usage)
    print(p)
    return 0


if __name__ == "__main__":
    sys.exit(main())
