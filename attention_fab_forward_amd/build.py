"""Build libfab.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m attention_fab_forward_amd.build [--jobs N]
Objects go to _build/ at the repository root; the shared library is written
next to this file so the Python binding can load it in-tree.
"""
import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libfab.so")
BUILD = os.path.join(ROOT, "_build")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unknown-pragmas",
    # keep packed-fp32 instructions out of device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source extra flags.  The attention kernels keep MFMA accumulators in
# arch VGPRs (their softmax / gradient math reads them every step; AGPR
# residency would add a copy per element).  The GeLU MLP kernels ask for the
# same; the forward's 64-row output block still overflows into AGPRs, while
# its partial H tiles no longer pass through them (forward and dC about 4 %
# faster, alternating runs).
FILE_FLAGS = {
    "attn_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "attn_f32_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "mlp.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libfab.so")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src, build_dir, defines):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    extra = FILE_FLAGS.get(os.path.basename(src), [])
    cmd = [hipcc(), *FLAGS, *extra, *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = [ln for ln in res.stderr.splitlines()
             if "packed-fp32-ops" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(noise))
    return obj, noise


def build(jobs=None, verbose=False, out=OUT, defines=(), build_dir=BUILD):
    """Compile every source in csrc/ and link libfab.so; returns its path.

    `defines` are extra preprocessor definitions (tile-shape experiments write
    their library to another `out` path)."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, build_dir, defines), srcs))
    objs = [r[0] for r in results]
    if verbose:
        for _, noise in results:
            for ln in noise:
                print(ln, file=sys.stderr)
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link of libfab.so failed:\n" + res.stderr)
    os.replace(tmp, out)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    main()
