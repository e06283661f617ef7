"""Build the gfx950 HIP library ``libkvq.so`` in-tree with hipcc.

Usage: ``python -m int4_quantized_kv_amd.build`` (or ``build()`` from Python).
Every HIP translation unit under ``csrc/`` is compiled for gfx950 only and linked into
one shared library next to this file, where the Python binding loads it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libkvq.so")
BUILD_DIR = os.path.join(HERE, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

SOURCES = ["api.hip", "quant.hip", "codec.hip", "decode.hip", "decode_mfma.hip"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no fused multiply-add contraction: every fma in the kernels is written out, so
    # the quantizers' rounding sequence is exactly the one checked on the host
    "-ffp-contract=off",
    # packed fp32 ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs (no AGPR copies around the softmax rescale)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # atomics stay single-lane as written (the optimizer's wave-combining rewrite reads
    # each result back at once, which waits for every transfer in flight)
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall",
    "-Wno-unused-function",
]


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        noisy = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write("\n".join(noisy) + "\n")
        elif verbose and noisy:
            print("\n".join(noisy))
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        sys.stderr.write(r.stdout.decode(errors="replace"))
        raise RuntimeError("link of libkvq.so failed")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
