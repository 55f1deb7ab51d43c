"""Build liblpfa.so in-tree with hipcc for gfx950 (python -m precision_attention_mxfp8_amd.build)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["quant.hip", "attn_fwd.hip", "attn_bwd.hip", "abi.cpp", "validate.cpp"]
OUTPUT = os.path.join(PKG, "liblpfa.so")
# measured-ceiling microbenchmarks for the benchmark's roofline fractions (not part of the C ABI)
PEAK_SOURCE = "peak.hip"
PEAK_OUTPUT = os.path.join(PKG, "libpeak.so")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build_command(output: str = OUTPUT, sources=None):
    sources = SOURCES if sources is None else sources
    return [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed FP32 VALU ops stay off: scalar float code only
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # no kernel produces NaN from in-domain (finite) inputs; infinities stay honoured. Lets
            # fmaxf skip NaN canonicalisation in the softmax.
            "-fno-honor-nans",
            # matrix-instruction results in VGPRs: the softmax reads the score tiles with VALU ops,
            # and AGPR results would cost one v_accvgpr_read per element.
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            # keep matrix instructions where they are written: sinking them toward their uses
            # (past the attention loop's load-issue code) keeps every operand fragment alive at
            # once and spills the two-group loop
            "-mllvm", "-disable-machine-sink",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", output] + \
           [os.path.join(CSRC, s) for s in sources]


def _compile(output: str, sources, verbose: bool) -> None:
    tmp = output + ".tmp"
    cmd = build_command(tmp, sources)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, output)


def build_library(verbose: bool = False) -> str:
    """Compile every source into liblpfa.so, and the ceiling microbenchmarks into libpeak.so
    (always recompiles). Returns the product library's path."""
    _compile(OUTPUT, SOURCES, verbose)
    _compile(PEAK_OUTPUT, [PEAK_SOURCE], verbose)
    return OUTPUT


if __name__ == "__main__":
    print(build_library(verbose=True))
