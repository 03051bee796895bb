"""Compile the HIP sources of the library into int4_compressed_domain_amd/libtq.so (gfx950),
and the streaming-read probe (a measurement aid) into libtq_probe.so beside it.

Every source is compiled with -Xclang -target-feature -Xclang -packed-fp32-ops, so the
compiler emits no packed fp32 arithmetic. The append and dequantize kernels, whose codes
must be bit-identical to a sequential definition, additionally use -ffp-contract=off.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libtq.so")
PROBE_OUT = os.path.join(HERE, "libtq_probe.so")  # the measurement aid, apart from the method
BUILD = os.path.join(ROOT, "_build")
ARCH = os.environ.get("TQ_OFFLOAD_ARCH", "gfx950")

SOURCES = {
    "tq_api.hip": [],
    "append.hip": ["-ffp-contract=off"],
    "dequant.hip": ["-ffp-contract=off"],
    "decode.hip": [],
    "dense.hip": [],
}
PROBE_SOURCES = {"stream_read.hip": []}
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def build(verbose=False):
    """Compile libtq.so and libtq_probe.so; returns the path of libtq.so."""
    _link(_compile(SOURCES, verbose), OUT)
    _link(_compile(PROBE_SOURCES, verbose), PROBE_OUT)
    return OUT


def _compile(sources, verbose):
    os.makedirs(BUILD, exist_ok=True)
    procs, objs = [], []
    for src, extra in sources.items():
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + extra
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature name; that warning is noise
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if p.returncode != 0:
            failed.append(src)
            print("\n".join(lines), file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    return objs


def _link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    subprocess.check_call(cmd)
    os.replace(tmp, out)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
