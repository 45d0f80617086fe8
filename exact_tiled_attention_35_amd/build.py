"""Build the HIP library in-tree: ``python -m exact_tiled_attention_35_amd.build``.

Compiles ``csrc/attn_api.hip``, ``csrc/attn_bwd_api.hip`` and
``csrc/attn_decode_api.hip`` (C ABI + kernels) for gfx950, one hipcc per
source in parallel, and links them into ``libattn.so`` next to this file, and writes the compiler's per-kernel
resource report (VGPRs, AGPRs, LDS, scratch, occupancy) to
``_build/resource_usage.txt``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_NAME = "libattn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
BUILD_DIR = os.path.join(PKG, "_build")
SOURCES = [os.path.join(PKG, "csrc", n) for n in ("attn_api.hip", "attn_bwd_api.hip", "attn_decode_api.hip")]
HEADERS = [os.path.join(PKG, "csrc", n) for n in ("gfx950_ops.hpp", "attn_fwd_kernel.hpp",
                                                  "attn_fwd_splitk_kernel.hpp",
                                                  "attn_fwd_k16_kernel.hpp",
                                                  "attn_bwd_kernel.hpp", "attn_decode_kernel.hpp",
                                                  "attn_host.hpp")] + [
    os.path.join(ROOT, "include", "attn.h")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_flags() -> list:
    return [
        "--offload-arch=gfx950",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        # Packed fp32 VALU ops are kept out of the generated code.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # Device code only: no NaN operands are expected, so max() needs no
        # NaN-quieting copies of its inputs.
        "-Xarch_device", "-fno-honor-nans",
        # Keep MFMA accumulators in architectural VGPRs (the softmax reads and
        # rescales them with VALU instructions; AGPR copies would cost more).
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-I", os.path.join(ROOT, "include"),
        "-I", os.path.join(PKG, "csrc"),
    ]


def build_library(verbose: bool = False) -> str:
    """Compile each source to an object in parallel (one hipcc per source),
    then link the shared library."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(BUILD_DIR, exist_ok=True)
    flags = [f for f in compile_flags() if f != "-shared"]
    objs = [os.path.join(BUILD_DIR, os.path.basename(src) + ".o") for src in SOURCES]

    def compile_one(src, obj):
        cmd = [hipcc()] + flags + ["-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        return subprocess.run(cmd, capture_output=True, text=True)

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        procs = list(ex.map(compile_one, SOURCES, objs))
    report = os.path.join(BUILD_DIR, "resource_usage.txt")
    with open(report, "w") as f:
        for p in procs:
            f.write(p.stderr)
    for p in procs:
        if p.returncode != 0:
            errors = [ln for ln in p.stderr.splitlines() if "error" in ln]
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors[:40] or p.stderr.splitlines()[-40:]))
    tmp = LIB_PATH + ".tmp"
    link = subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp],
                          capture_output=True, text=True)
    if link.returncode != 0:
        raise RuntimeError("link failed:\n" + link.stderr[-4000:])
    os.replace(tmp, LIB_PATH)
    write_build_info()
    return LIB_PATH


BUILD_INFO = os.path.join(PKG, "libattn.build.json")


def write_build_info() -> None:
    """Record, beside the library, the git revision of the tree it was built
    from (with "+modified" when tracked files differ from it), so that a run
    on a copy of the tree without its .git can still name the build."""
    import json

    rev = None
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"],
                           capture_output=True, text=True, timeout=10)
        if r.returncode == 0:
            rev = r.stdout.strip()
            d = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--untracked-files=no"],
                               capture_output=True, text=True, timeout=10)
            if d.returncode == 0 and d.stdout.strip():
                rev += "+modified"
    except (OSError, subprocess.SubprocessError):
        pass
    with open(BUILD_INFO, "w") as f:
        json.dump({"git_rev": rev}, f)


if __name__ == "__main__":
    path = build_library(verbose="-v" in sys.argv)
    print(path)
