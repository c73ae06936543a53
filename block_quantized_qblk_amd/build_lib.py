"""Build libqblk.so (gfx950) in-tree with hipcc.

    python -m block_quantized_qblk_amd.build_lib [--changed]

Objects go to <repo>/_build/, the shared library next to this file.
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
LIB = os.path.join(PKG, "libqblk.so")

ARCH = "gfx950"

SOURCES = [
    "quantize_act.hip",
    "pack_weights.hip",
    "gemv.hip",
    "gemv_select.cpp",
    "gemv_float.hip",
    "gemm.hip",
    "gemm_small.hip",
    "block_sums.hip",
    "kv.hip",
    "api.cpp",
]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    f"--offload-arch={ARCH}",
    # no packed-fp32 VALU instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep fp32 denormals (the quantizers' decisions must match IEEE)
    "-fno-gpu-flush-denormals-to-zero",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


# per-source extra flags: the GEMM's MFMA results feed VALU instructions
# directly, so MFMAs write VGPRs instead of accumulation registers (no copy
# back per result)
EXTRA = {"gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "gemm_small.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build libqblk.so")
    return exe


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + EXTRA.get(src, [])
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _stale(src):
    """Whether src's object is missing or older than src or any header."""
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if not os.path.exists(obj):
        return True
    deps = [os.path.join(CSRC, src)] + [os.path.join(d, f) for d in (CSRC, os.path.join(ROOT, "include"))
                                        for f in os.listdir(d) if f.endswith(".h")]
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) > t for d in deps)


def build(verbose=True, changed_only=False):
    """Compile the sources and link libqblk.so. Recompiles every source
    unless changed_only (then only those whose object is older than the
    source or a header)."""
    os.makedirs(BUILD, exist_ok=True)
    todo = [s for s in SOURCES if not changed_only or _stale(s)]
    jobs = min(max(1, len(todo)), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(_compile, todo))
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-o", tmp] + objs + [f"--offload-arch={ARCH}", "-fPIC"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(changed_only="--changed" in sys.argv[1:])
