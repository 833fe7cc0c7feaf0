"""Build libmxattn.so in place: every source under csrc/ compiled by hipcc for
gfx950, then linked into one shared library next to this file.

    python -m bit_microscaled_flashattention_amd.build [--jobs N] [--verbose]
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmxattn.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "quantize.hip", "prefill.hip", "decode.hip", "select.hip", "gather.hip"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # No packed fp32 (v_pk_*_f32) instructions are generated.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # fp32 subnormals are kept: the quantiser must code them exactly.
    "-fno-gpu-flush-denormals-to-zero",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
]


# Per-source additions.  The attention kernel's logits are finite or -inf
# (masked keys) and never NaN, so max/min need no NaN canonicalisation.  The
# selection kernels keep their MFMA results in VGPRs: with accumulators in
# AGPRs the column-mass loop copied every logit out before its exponential.
EXTRA = {"prefill.hip": ["-fno-honor-nans"],
         "select.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libmxattn.so")
    return path


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    return obj, msgs


def build(jobs=None, verbose=False):
    """Compile every source and link libmxattn.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    for (obj, msgs) in results:
        if msgs and verbose:
            print(msgs)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    sys.exit(main())
