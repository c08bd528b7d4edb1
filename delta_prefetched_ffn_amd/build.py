"""Builds libnp.so (the HIP library behind include/np.h) for gfx950 with hipcc.

Usage: python -m delta_prefetched_ffn_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libnp.so")
SOURCES = ["np_api.hip", "k_delta.hip", "k_scatter.hip", "k_ffn.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off: scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str, obj_dir: str) -> str:
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    obj_dir = os.path.join(ROOT, "_build", "np")
    os.makedirs(obj_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir), SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", flush=True)
    return LIB


# Host-side sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer on the host code only;
# the gfx950 device code is built as usual): each -fsanitize= goes behind -Xarch_host.
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LIB = os.path.join(ROOT, "_build", "san", "libnp_san.so")


def build_sanitized(force: bool = False) -> str:
    """libnp with sanitized host code into _build/san/libnp_san.so (rebuilt when a source is newer).
    A process loading it needs the clang ASan runtime preloaded (sanitizer_runtime())."""
    obj_dir = os.path.dirname(SAN_LIB)
    os.makedirs(obj_dir, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(CSRC, "np_internal.hpp"),
                                                      os.path.join(INCLUDE, "np.h")]
    if not force and os.path.exists(SAN_LIB) and os.path.getmtime(SAN_LIB) >= max(map(os.path.getmtime, srcs)):
        return SAN_LIB

    def comp(src):
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *[f for f in FLAGS if f != "-O3"], "-O1", "-g", *SAN_HOST, "-c", os.path.join(CSRC, src),
               "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(comp, SOURCES))
    tmp = SAN_LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN_HOST, "-Xarch_host", "-shared-libasan", "-o",
           tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def sanitizer_runtime() -> str:
    """The shared ASan (+UBSan) runtime of the ROCm clang that the sanitized builds link against."""
    r = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        import glob
        found = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        path = found[0] if found else ""
    return path


if __name__ == "__main__":
    build()
    sys.exit(0)
