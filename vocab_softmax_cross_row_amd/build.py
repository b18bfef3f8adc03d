"""Build libvocab_ce.so (HIP, gfx950) in-tree with hipcc.

    python -m vocab_softmax_cross_row_amd.build [-v]

Packed fp32 instructions are turned off for all device code
(``-packed-fp32-ops``); the host pass warns that it does not know the
feature, which is harmless.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libvocab_ce.so")
SOURCES = [os.path.join(CSRC, f) for f in ("ce_kernels.hip", "ce_fused.hip", "ce_linear.hip", "ce_api.hip")]
ARCH = "gfx950"


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def build(verbose: bool = False) -> str:
    # the e^z table of the smoothed bf16 statistics, compiled into the code object
    subprocess.run([sys.executable, os.path.join(CSRC, "gen_exp_table.py"),
                    os.path.join(CSRC, "ce_exp_table.inc")], check=True, capture_output=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-I", INCLUDE, "-I", CSRC, "-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
