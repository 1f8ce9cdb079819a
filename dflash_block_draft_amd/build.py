"""Build the gfx950 HIP library libdflash_mla.so in-tree with hipcc.

Every source in csrc/ is compiled to an object for gfx950 only, then linked
into one shared library next to this file.  Packed-fp32 VALU forms are
disabled for device code (-packed-fp32-ops); hipcc's host pass warns that it
does not know that feature, which is expected.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdflash_mla.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(HERE, "..", "include"),
]


# Per-source device flags.  The backward kernels keep 160 accumulator registers
# (dK, dV or dQ) plus register-resident operands; letting the MFMAs write their
# score tiles to ordinary VGPRs (which the softmax reads anyway) instead of
# accumulator registers avoids spilling.
#
# The GQA block attention rescales its output accumulators on the vector unit;
# in VGPR form they need no copies out of and back into accumulator registers.
FILE_FLAGS = {
    # The forward key loop's exact path is rare; placing those blocks after the
    # loop keeps the common path free of jumps over them.
    "attn_bf16.hip": ["-mllvm", "-force-loop-cold-block"],
    "attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "gqa.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(hipcc: str, src: str, extra, build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc, *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = True, extra_flags=()) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s, list(extra_flags)), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


# Host-side sanitizer build of the C ABI layer (argument checks, layouts,
# dispatch): abi.hip's host code is compiled with AddressSanitizer and
# UndefinedBehaviorSanitizer (device code untouched: each -fsanitize applies to
# the host pass only), the other objects come from the regular build.  Loading
# it needs the ASan runtime preloaded (san_runtime()).
SAN_BUILD = os.path.join(HERE, "_build_san")
SAN_LIB = os.path.join(SAN_BUILD, "libdflash_mla_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]


def san_runtime() -> str:
    """The clang AddressSanitizer runtime matching hipcc's compiler."""
    root = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(_hipcc()))), "llvm", "lib", "clang")
    for ver in sorted(os.listdir(root), reverse=True):
        p = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    raise RuntimeError("the clang ASan runtime is not installed")


def build_sanitized(verbose: bool = True) -> str:
    hipcc = _hipcc()
    if not os.path.exists(LIB):
        build(verbose=verbose)
    os.makedirs(SAN_BUILD, exist_ok=True)
    abi = os.path.join(CSRC, "abi.hip")
    san_obj = _compile(hipcc, abi, SAN_FLAGS, SAN_BUILD)
    objs = [san_obj] + [os.path.join(BUILD, os.path.basename(s) + ".o") for s in sources() if s != abi]
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-shared-libasan",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", *objs, "-o", SAN_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB} (host ASan + UBSan on abi.hip)")
    return SAN_LIB


if __name__ == "__main__":
    build()
