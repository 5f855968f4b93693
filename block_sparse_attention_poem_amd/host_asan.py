"""Host AddressSanitizer check of libpoem's C ABI layer (CPU only; no GPU needed).

Builds a second copy of the library whose host code is instrumented by ASan (the
argument validation, geometry and workspace layout of poem_api.cpp and the launch
code of the .hip files; device code is compiled as usual) and runs the host-side
API tests against it, with the sanitizer runtime preloaded into Python:

    python -m block_sparse_attention_poem_amd.host_asan

Every invalid-argument path of the C ABI is exercised there, so an out-of-bounds
read of a host array (sequence lengths, thresholds) or a use of a stale buffer in
the error path shows up as a sanitizer report and a failing exit status. Leak
checking is off: the Python interpreter itself is not instrumented.
"""
import glob
import os
import subprocess
import sys

from . import build as B

OUT_DIR = os.path.join(B.PKG, "_build", "asan")
OUT = os.path.join(OUT_DIR, "libpoem_asan.so")


def runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("clang's ASan runtime (libclang_rt.asan-x86_64.so) not found under /opt/rocm/llvm")
    return found[-1]


def build_asan():
    os.makedirs(OUT_DIR, exist_ok=True)
    cc = B.hipcc()
    sanitize = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = []
    for src in B.SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        cmd = [cc] + B.flags() + sanitize + ["-c", os.path.join(B.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        objs.append(obj)
    cmd = [cc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-shared-libasan", "-Xarch_host", "-fsanitize=address",
           "-o", OUT] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    return OUT


def main():
    lib = build_asan()
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    if "__asan_report" not in nm:
        raise RuntimeError(f"{lib} carries no ASan instrumentation")
    env = dict(os.environ)
    env["POEM_LIB"] = lib
    env["LD_PRELOAD"] = runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", os.path.join(B.ROOT, "tests", "test_host_api.py")]
    print("POEM_LIB=%s LD_PRELOAD=%s %s" % (lib, env["LD_PRELOAD"], " ".join(cmd)), flush=True)
    return subprocess.run(cmd, env=env, cwd=B.ROOT).returncode


if __name__ == "__main__":
    sys.exit(main())
