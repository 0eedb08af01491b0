"""Build the HIP library libfa.so in-tree with hipcc for gfx950.

Every .hip file under csrc/ is compiled to an object (in parallel), then the
objects are linked into tiled_attention_fa_amd/libfa.so.  Packed fp32 VALU
instructions are switched off for device code; no fast-math flags are used
(the kernels rely on -inf masks and exp2(-inf) = 0).
"""

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # keep MFMA accumulators in VGPRs: the softmax reads every score
            # with VALU instructions, which cannot take AGPR operands
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            f"-I{INCLUDE}", f"-I{CSRC}"]


TUNE_LIB = os.path.join(PKG, "libfa_tune.so")
TUNE_DIR = os.path.join(BUILD_DIR, "tune")


def _compile(src: str, extra, out_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *common_flags(), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    lines = [ln for ln in (r.stdout + r.stderr).splitlines()
             if "packed-fp32-ops' is not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(lines))
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build(jobs: int = 0, extra=(), tune: bool = True) -> str:
    """Compile and link libfa.so and (with tune) the tile-calibration
    library libfa_tune.so, the same sources with every workgroup shape of
    the sweep instantiated (-DFA_TILE_SWEEP).  Returns the path of
    libfa.so.  Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(TUNE_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    work = [(s, list(extra), BUILD_DIR) for s in srcs]
    if tune:
        work += [(s, list(extra) + ["-DFA_TILE_SWEEP"], TUNE_DIR) for s in srcs]
    # the largest translation units first, so the pool ends together
    work.sort(key=lambda w: -os.path.getsize(w[0]) - (1 << 20) * ("FA_TILE_SWEEP" in w[1] and "mfma" in w[0]))
    jobs = jobs or min(len(work), os.cpu_count() or 4, 16)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda w: _compile(*w), work))
    _link([o for o, w in zip(objs, work) if w[2] == BUILD_DIR], LIB)
    if tune:
        _link([o for o, w in zip(objs, work) if w[2] == TUNE_DIR], TUNE_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
