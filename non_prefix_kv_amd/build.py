"""Builds libcacheblend.so in-tree with hipcc for gfx950.

Usage: python non_prefix_kv_amd/build.py   (or __graft_entry__.build()); run it by
path: importing the package itself loads the built library.
Every source is compiled each time (parallel hipcc processes), then linked.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libcacheblend.so")
OBJ_DIR = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
    "-Wno-unused-result",
]


# Host code built again with AddressSanitizer and UndefinedBehaviorSanitizer
# (host side only: each flag after -Xarch_host; the GPU code is unchanged),
# for the CPU tests of the host-only entry points.
SAN_OUT = os.path.join(PKG, "_build_san", "libcacheblend_san.so")
SAN_FLAGS = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
             "-fno-omit-frame-pointer"]


def _compile(src, san=False):
    odir = os.path.dirname(SAN_OUT) if san else OBJ_DIR
    obj = os.path.join(odir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *(SAN_FLAGS if san else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj, err


def _link(objs, out, extra=()):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)


def build(verbose=True, sanitized=True):
    os.makedirs(OBJ_DIR, exist_ok=True)
    os.makedirs(os.path.dirname(SAN_OUT), exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = max(1, int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(jobs) as ex:
        plain = [ex.submit(_compile, src) for src in srcs]
        san = [ex.submit(_compile, src, True) for src in srcs] if sanitized else []
        results = [f.result() for f in plain]
        san_results = [f.result() for f in san]
    for obj, err in results:
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    _link([o for o, _ in results], OUT)
    if sanitized:
        # the sanitizer runtimes are not linked into a shared library: they
        # come from the ASan runtime preloaded by the process that loads it
        _link([o for o, _ in san_results], SAN_OUT)
    if verbose:
        print(f"built {OUT}" + (f" and {SAN_OUT}" if sanitized else ""))
    return OUT


if __name__ == "__main__":
    build()
