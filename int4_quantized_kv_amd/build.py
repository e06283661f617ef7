"""Build the gfx950 HIP library ``libkvq.so`` in-tree with hipcc.

Usage: ``python -m int4_quantized_kv_amd.build`` (or ``build()`` from Python).
Every HIP translation unit under ``csrc/`` is compiled for gfx950 only and linked into
one shared library next to this file, where the Python binding loads it.
"""
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libkvq.so")
# the benchmark's streaming-read reference (not part of the library's ABI)
BENCH_OUT = os.path.join(HERE, "libkvq_bench.so")
BENCH_SOURCES = ["stream_read.hip"]
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


# Sources whose kernels count their own global->LDS transfers with explicit vmcnt waits:
# a register spill there would put scratch loads and stores into the same counter and
# break those waits, so the build reports every kernel's scratch use and fails on any.
NO_SCRATCH = {"decode_mfma.hip"}
RESOURCE_REMARKS = ["-Rpass-analysis=kernel-resource-usage"]


def _scratch_users(text):
    """Kernels with a nonzero scratch size in the compiler's resource-usage remarks."""
    users, name = [], None
    for ln in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", ln)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", ln)
        if m and int(m.group(1)) > 0:
            users.append(f"{name} ({m.group(1)} bytes/lane)")
    return users


# The timeline probe: the same sources built with -DKVQ_TIMELINE, where the matrix-core
# decode kernel records the real-time counter at its phase points (bench.py --timeline).
# Built on request only (python -m int4_quantized_kv_amd.build --timeline).
TIMELINE_OUT = os.path.join(HERE, "libkvq_timeline.so")


def build(verbose=False, timeline=False):
    bdir = os.path.join(BUILD_DIR, "timeline") if timeline else BUILD_DIR
    os.makedirs(bdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, *(["-DKVQ_TIMELINE"] if timeline else []),
               *(RESOURCE_REMARKS if src in NO_SCRATCH else []), "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        noisy = [ln for ln in text.splitlines()
                 if "packed-fp32-ops" not in ln and "kernel-resource-usage" not in ln]
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write("\n".join(noisy) + "\n")
            continue
        if verbose and noisy:
            print("\n".join(noisy))
        if src in NO_SCRATCH:
            users = _scratch_users(text)
            if users:
                failed.append(src)
                sys.stderr.write(src + ": kernels using scratch memory:\n  " + "\n  ".join(users) + "\n")
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    if timeline:
        _link(objs, TIMELINE_OUT)
        return TIMELINE_OUT
    _link(objs, OUT)
    bench_objs = []
    for src in BENCH_SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        r = subprocess.run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj],
                           stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if r.returncode != 0:
            sys.stderr.write(r.stdout.decode(errors="replace"))
            raise RuntimeError("hipcc failed for: " + src)
        bench_objs.append(obj)
    _link(bench_objs, BENCH_OUT)
    return OUT


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        sys.stderr.write(r.stdout.decode(errors="replace"))
        raise RuntimeError("link of " + os.path.basename(out) + " failed")
    os.replace(tmp, out)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, timeline="--timeline" in sys.argv))
