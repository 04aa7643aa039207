"""Build libhybattn.so (the HIP library) in-tree for gfx950 with hipcc.

Every call recompiles: each ``csrc/*.hip`` file to an object under
``_build/`` (in parallel), then one shared-library link into the package
directory.  Run ``python -m hybrid_softmax_linear_block_amd.build_lib``.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libhybattn.so")

ARCH = "gfx950"
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the same
# sources (device code is compiled as usual), for running the C-ABI checks
# on the CPU: build(sanitize=True) writes _build/san/libhybattn.so.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
SAN_LIB = os.path.join(BUILD, "san", "libhybattn.so")


def asan_runtime():
    """Path of clang's shared AddressSanitizer runtime (to preload into a
    host process that loads the sanitized library)."""
    root = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(_hipcc()))), "llvm", "lib", "clang")
    for ver in sorted(os.listdir(root), reverse=True) if os.path.isdir(root) else []:
        p = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    raise RuntimeError("libclang_rt.asan-x86_64.so not found under " + root)


def _compile(src, hipcc, extra, build=BUILD):
    obj = os.path.join(build, os.path.basename(src) + ".o")
    cmd = [hipcc] + FLAGS + extra + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr[-8000:]))
    return obj


def build(verbose=False, extra=(), sanitize=False):
    hipcc = _hipcc()
    out_dir = os.path.join(BUILD, "san") if sanitize else BUILD
    lib = SAN_LIB if sanitize else LIB
    flags = list(extra) + (SANITIZE if sanitize else [])
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    jobs = min(8, len(srcs), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, flags, out_dir), srcs))
    tmp = lib + ".tmp"
    link = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"] \
        if sanitize else []
    cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + link + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr[-8000:])
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
