"""Build libhsa_attn.so for gfx950 in-tree with hipcc (no JIT cache).

    python -m long_context_hybrid_kv_amd.build              # libhsa_attn.so
    python -m long_context_hybrid_kv_amd.build --sanitize   # libhsa_attn_san.so

Every HIP source under csrc/ is compiled for gfx950 and linked into
long_context_hybrid_kv_amd/libhsa_attn.so.  Packed fp32 instructions are
disabled (-packed-fp32-ops); sources are compiled in parallel.

--sanitize builds the same library with AddressSanitizer and
UndefinedBehaviorSanitizer in its host code only (argument checks, workspace
carving, launch set-up; the GPU code is built as usual) into
libhsa_attn_san.so, linked against the shared sanitizer runtime: a process
that loads it preloads that runtime (sanitizer_runtime() names it) and points
the binding at the library with HSA_ATTN_LIB.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libhsa_attn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-result",
]


# per-source additions: the attention kernel keeps its MFMA accumulators in
# ordinary VGPRs (no copies between accumulation and arithmetic registers when
# the online softmax rescales them)
EXTRA = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


# host-only sanitizers: each -fsanitize= applies to the host pass alone
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
SAN_OBJ = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(PKG, "libhsa_attn_san.so")


def sanitizer_runtime() -> str:
    """Path of the shared AddressSanitizer runtime of hipcc's clang."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True, check=True)
    return r.stdout.strip().splitlines()[-1]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, obj_dir: str = OBJ, extra=()) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True, sanitize: bool = False) -> str:
    obj_dir, lib = (SAN_OBJ, SAN_LIB) if sanitize else (OBJ, LIB)
    extra = SAN_FLAGS if sanitize else []
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, extra), srcs))
    tmp = lib + ".tmp"
    link_extra = ["-shared-libsan", *SAN_FLAGS] if sanitize else []
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
