"""Build libmla.so (hand-written HIP for gfx950) in the package directory.

    python -m mla_latent_kv_19_amd.build

Compiles every csrc/*.hip and csrc/*.cpp with hipcc and links one shared
library.  Packed fp32 instructions are disabled for all device code.
"""

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmla.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: libmla.so cannot be built")
    return path


# Per-file extra flags.  decode.hip keeps all 256 AGPRs for its output
# accumulators (written by inline-asm MFMAs) and needs the compiler's own MFMAs
# (the score product) to accumulate in VGPRs.
EXTRA_FLAGS = {
    "decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def build(verbose=False):
    """Compile all sources and link libmla.so; returns the library path."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    objs = []
    procs = []
    for src in sources:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        extra = EXTRA_FLAGS.get(os.path.basename(src), [])
        cmd = [hipcc(), *HIPCC_FLAGS, *extra, *lang, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd))
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature flag; that note is harmless.
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if p.returncode != 0:
            failed.append((src, "\n".join(lines)))
        elif lines and verbose:
            print("\n".join(lines))
    if failed:
        msg = "\n\n".join(f"{s}:\n{t}" for s, t in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
