"""Compile libtrace_quant.so for gfx950 with hipcc (in-tree)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", "trace_quant.hip"), os.path.join(HERE, "csrc", "trace_record.cpp")]
OUT = os.path.join(HERE, "libtrace_quant.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-shared",
    "-ffp-contract=off",                       # no fused multiply-add in the scale chain
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


# The measurement build of the one-pass phase clocks (phase_clock.py): the
# same sources and flags with TRACE_OP_PHASE_CLOCK=1.  Not the product library.
OUT_PHASE_CLOCK = os.path.join(HERE, "libtrace_quant_phaseclock.so")


def build(verbose=False, out=OUT, defines=()):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *["-D" + d for d in defines], "-I", os.path.join(ROOT, "include"), *SRCS,
           "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd))
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, out)
    return out


def build_phase_clock(verbose=False):
    return build(verbose, OUT_PHASE_CLOCK, ("TRACE_OP_PHASE_CLOCK=1",))


if __name__ == "__main__":
    print(build(verbose=True))
