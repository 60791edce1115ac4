"""Build libdsa.so (the HIP library) in place for gfx950.

    python -m sparse_attention_14_amd.build        (or python sparse_attention_14_amd/build.py)

Every .hip file under csrc/ is compiled with hipcc --offload-arch=gfx950 into
sparse_attention_14_amd/libdsa.so.  Packed-FP32 instructions are disabled
(-target-feature -packed-fp32-ops).
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libdsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


# Per-file code-generation options.  index_scores.hip, prefill_scores.hip: MFMA
# results in ordinary VGPRs (not accumulation registers), so the score epilogue
# reads them without a v_accvgpr_read copy per element.
FILE_FLAGS = {"index_scores.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "prefill_scores.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = False, jobs: int = 4) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *flags, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    while procs:
        _wait(procs.pop(0))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", OUT + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


def _wait(item):
    cmd, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    # hipcc's host pass does not know the packed-fp32 feature; that warning is expected.
    lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
    if lines:
        print("\n".join(lines), flush=True)
    if p.returncode != 0:
        raise subprocess.CalledProcessError(p.returncode, cmd)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
