"""Build libspecverify.so (gfx950) in-tree with hipcc.

Every HIP source is compiled with packed-fp32 instruction selection disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``): the kernels use scalar
and MFMA fp32 arithmetic only.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libspecverify.so")
SOURCES = ["api.cpp", "accept.hip", "attn.hip", "compact.hip", "noalloc.hip", "lmhead.hip"]
ARCH = os.environ.get("SPECVERIFY_ARCH", "gfx950")


def hipcc_command(out=LIB):
    return (["hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-o", out] + [os.path.join(CSRC, s) for s in SOURCES])


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = hipcc_command(tmp)
    res = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
