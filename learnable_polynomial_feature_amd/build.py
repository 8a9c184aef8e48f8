"""Build libllops.so (all HIP kernels + the C ABI) for gfx950, in-tree.

    python -m learnable_polynomial_feature_amd.build
    python -m learnable_polynomial_feature_amd.build --host-sanitize

Every source is compiled by hipcc with packed-fp32 instruction selection
disabled, then linked into learnable_polynomial_feature_amd/libllops.so.
--host-sanitize builds libllops_hostsan.so instead: the same library with
AddressSanitizer and UndefinedBehaviorSanitizer on its host code only (every
-fsanitize behind -Xarch_host; the device code is unchanged). Load it with
LLOPS_LIBRARY set to its path and the ASan runtime preloaded, e.g.

    LD_PRELOAD=$(hipcc -print-file-name=libclang_rt.asan-x86_64.so) \
    ASAN_OPTIONS=detect_leaks=0 LLOPS_LIBRARY=<pkg>/libllops_hostsan.so \
    python -m pytest tests -m "not gpu" -k "abi or binding"
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libllops.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["featmap.hip", "featmap_bwd.hip", "attn.hip", "attn32.hip", "attn_bwd.hip", "decode.hip",
           "abi.cpp"]

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


# Per-source flags. The backward kernels hold MFMA accumulators and operands
# together in more than 256 registers; with MFMA results in VGPRs the
# allocator stops shuttling accumulators through AGPR copies every step.
EXTRA = {"featmap_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


# host code only: each -fsanitize applies to the host pass alone
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def _compile(src: str, build_dir: str = BUILD, extra: tuple = ()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[cmd.index("-c"):cmd.index("-c")] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l
                     and "not a recognized feature" not in l and l.strip())
    if warn:
        print(f"[build] {src}:\n{warn}", file=sys.stderr)
    return obj


def build(jobs: int = 4, host_sanitize: bool = False) -> str:
    build_dir = BUILD + ("_hostsan" if host_sanitize else "")
    lib = os.path.join(PKG, "libllops_hostsan.so") if host_sanitize else LIB
    extra = tuple(HOST_SAN) if host_sanitize else ()
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, extra), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-shared-libsan", *objs,
           "-o", tmp] if host_sanitize else [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC",
                                              *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(host_sanitize="--host-sanitize" in sys.argv[1:]))
