"""Build the HIP library ``libcfa.so`` in-tree with hipcc for gfx950.

    python -m causal_flashattention_amd.build        # or build() from Python

Each source under ``csrc/`` compiles to an object in ``_build/`` (in parallel), then one
shared library is linked next to this file. Always recompiles: a stale library is worse than a
slow build.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libcfa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off: the compiler must not form v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


# The attention kernels take no non-finite inputs (masked scores are -inf, never NaN), so they
# are built without NaN semantics and with the IEEE mode bit off: max/min then need no
# canonicalising instruction before each use of a matrix-core result. The quantiser keeps
# both, since it must detect NaN/Inf blocks.
NO_NAN_SOURCES = {"attn_fwd.hip", "attn_fwd_mx.hip", "attn_bwd_mx.hip"}
NO_NAN_FLAGS = ["-fno-honor-nans", "-mno-amdgpu-ieee"]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    extra = NO_NAN_FLAGS if os.path.basename(src) in NO_NAN_SOURCES else []
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    return obj, msgs


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    for obj, msgs in results:
        if verbose and msgs.strip():
            print(msgs)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
