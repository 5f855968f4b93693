"""Build libpoem.so in-tree for gfx950 with hipcc (no JIT, no site-packages install).

Usage: python -m block_sparse_attention_poem_amd.build [--debug]
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libpoem.so")
SOURCES = ["attn_fwd.hip", "selector.hip", "poem_api.cpp"]
# the on-card MFMA rate probe the benchmark reports beside the quoted peak (its own library)
PROBE_OUT = os.path.join(PKG, "libpoem_probe.so")
PROBE_SOURCES = ["mfma_probe.hip"]
ARCH = "gfx950"


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


def flags(debug=False):
    f = [f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-x", "hip",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC,
         # packed fp32 VALU ops stay off (hipcc's host pass warns that it does not know the feature)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    f += ["-O1", "-g"] if debug else ["-O3"]
    return f


def build(debug=False, verbose=False):
    os.makedirs(os.path.join(PKG, "_build"), exist_ok=True)
    cc = hipcc()
    objs = []

    def compile_one(src):
        obj = os.path.join(PKG, "_build", src + ".o")
        cmd = [cc] + flags(debug) + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES) + len(PROBE_SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES + PROBE_SOURCES))
    for out, o in ((OUT, objs[:len(SOURCES)]), (PROBE_OUT, objs[len(SOURCES):])):
        tmp = out + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + o
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stderr)
        os.replace(tmp, out)
    return OUT


if __name__ == "__main__":
    print(build(debug="--debug" in sys.argv, verbose=True))
