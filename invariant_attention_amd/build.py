"""Build step: compile ``csrc/bi_attn.hip``, ``csrc/bi_norm.hip`` and ``csrc/bi_gemm.hip`` for
gfx950 into ``libbiattn.so`` (in-tree)."""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", n) for n in ("bi_attn.hip", "bi_norm.hip", "bi_gemm.hip")]
OUT = os.path.join(HERE, "libbiattn.so")

# -ffp-contract=off: every fused multiply-add in the kernels is written out explicitly, so the
# compiler cannot contract the same source differently in the decode and prefill kernels.
# -packed-fp32-ops off: keep fp32 arithmetic on plain VALU instructions.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
    "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile the library (always recompiles) and return its path."""
    tmp = OUT + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *SRCS]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
