"""Build liblin.so (the HIP library) in-tree for gfx950 with hipcc.

Every kernel source is compiled on its own (in parallel), then linked into
memory_bound_weight_amd/liblin.so.  hipcc cross-compiles, so this runs on a
machine without a GPU.
"""
import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "liblin.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

# -packed-fp32-ops off: the compiler must not form v_pk_{add,mul,fma}_f32.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "lin_api.cpp")]


def _compile(src, extra):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = ["hipcc", "-x", "hip", "-c", src, "-o", obj] + FLAGS + extra
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stdout))
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in r.stdout.splitlines() if noise not in ln]
    return obj, "\n".join(msgs)


def build(extra_flags=(), jobs=None, verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, list(extra_flags)), srcs))
    for _, msg in results:
        if msg.strip() and verbose:
            print(msg)
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + \
        [o for o, _ in results]
    subprocess.check_call(cmd)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(extra_flags=sys.argv[1:], verbose=True))
