"""Build libvc.so (the HIP library behind include/vc.h) in-tree for gfx950.

    python -m kv_cache_compressed_amd.build        # compiles every csrc/*.hip and links libvc.so
    python -m kv_cache_compressed_amd.build --host-sanitize   # libvc_hostsan.so (ASan + UBSan host code)

Flags: -O3 for gfx950, no fast-math (the quantiser needs IEEE division and round-half-even), and
the packed-fp32 target feature disabled (the compiler must not emit packed fp32 arithmetic).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libvc.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in r.stderr.splitlines() if noise not in l and l.strip())
    if warn:
        print(warn, file=sys.stderr)
    return obj


HOSTSAN = os.path.join(PKG, "libvc_hostsan.so")
# AddressSanitizer + UndefinedBehaviorSanitizer on the host code of api.hip (argument validation,
# workspace sizing, launch set-up); device code and the other objects are the normal build's.
SAN_FLAGS = [f for s in ("address", "undefined") for f in ("-Xarch_host", f"-fsanitize={s}")] + [
    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def asan_runtime() -> str | None:
    """The clang AddressSanitizer runtime a sanitized library needs preloaded, if installed."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    root = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang")
    for ver in sorted(os.listdir(root)) if os.path.isdir(root) else []:
        cand = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(cand):
            return cand
    return None


def build_host_sanitized(verbose: bool = True) -> str:
    """libvc_hostsan.so: the normal objects with api.hip's host code rebuilt under ASan + UBSan.
    Load it with the ASan runtime preloaded (LD_PRELOAD=asan_runtime()) and VC_LIB pointing at it."""
    objs = [o for o in (os.path.join(BUILD, os.path.basename(f)[:-4] + ".o") for f in sources())]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        build(verbose=False)
    api = os.path.join(CSRC, "api.hip")
    san_obj = os.path.join(BUILD, "api_hostsan.o")
    cmd = [HIPCC, *FLAGS, *SAN_FLAGS, "-c", api, "-o", san_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    objs = [san_obj if os.path.basename(o) == "api.o" else o for o in objs]
    tmp = HOSTSAN + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, HOSTSAN)
    if verbose:
        print(f"built {HOSTSAN}")
    return HOSTSAN


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    if "--host-sanitize" in sys.argv[1:]:
        build_host_sanitized()
    else:
        build()
