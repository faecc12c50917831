"""Build libswr.so (the HIP library behind include/swr.h) for gfx950 in-tree.

    python sliding_window_ring_amd/build.py

Compiles each source with hipcc into sliding_window_ring_amd/_build/ and links
sliding_window_ring_amd/libswr.so.  Always recompiles (the build is the check
that the code compiles).

    python sliding_window_ring_amd/build.py --sanitize

builds the same library with AddressSanitizer and UndefinedBehaviorSanitizer
on its host code only (each -fsanitize= behind -Xarch_host; device code is
built as usual) into _build_san/libswr_san.so, for the CPU tests of the
validation and pool code (tests/test_sanitizers.py).  Loading it needs the
compiler's ASan runtime preloaded (sanitizer_runtime()).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libswr.so")
SOURCES = ["attn.hip", "chunked.hip", "append.hip", "gather.hip", "read_ceiling.hip", "noalloc.hip", "swr_api.cpp"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


SAN_DIR = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(SAN_DIR, "libswr_san.so")
# host-side sanitizers, each flag behind -Xarch_host so that no device code is
# instrumented
SAN_FLAGS = []
for _f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-g"):
    SAN_FLAGS += ["-Xarch_host", _f]


def _compile(src: str, extra, out_dir: str = OUT_DIR) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *CFLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; that line is noise
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in r.stdout.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(extra_flags=(), out: str = LIB, verbose: bool = True, out_dir: str = OUT_DIR, link_flags=()) -> str:
    os.makedirs(out_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags), out_dir), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *link_flags, *objs, "-o", tmp])
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def build_sanitized(force: bool = False) -> str:
    """libswr_san.so: host code under ASan + UBSan (rebuilt when a source is
    newer than it)."""
    srcs = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(ROOT, "include", "swr.h")]
    if force or not os.path.exists(SAN_LIB) or os.path.getmtime(SAN_LIB) < max(map(os.path.getmtime, srcs)):
        build(SAN_FLAGS, SAN_LIB, verbose=False, out_dir=SAN_DIR, link_flags=SAN_FLAGS)
    return SAN_LIB


def sanitizer_runtime() -> str:
    """Path of the ASan runtime of hipcc's compiler (it carries the UBSan
    handlers too), for LD_PRELOAD into an uninstrumented Python."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                         text=True, check=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        raise FileNotFoundError("clang's ASan runtime not found")
    return out


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        print(build_sanitized(force=True))
    else:
        build(sys.argv[1:])
