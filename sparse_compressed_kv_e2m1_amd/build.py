"""Build the gfx950 HIP library libsckv.so in-tree with hipcc.

Flags:
  --offload-arch=gfx950           CDNA4 only
  -ffp-contract=off               no implicit multiply-add fusion (bit-exact score/quant paths)
  -fgpu-flush-denormals-to-zero off (explicitly -fno-...): keep binary32 subnormals
  -fhip-fp32-correctly-rounded-divide-sqrt: IEEE division where '/' is used
  -Xclang -target-feature -Xclang -packed-fp32-ops (minus sign): no packed fp32 ops
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsckv.so")
SOURCES = ["abi.hip", "quant.hip", "rope.hip", "window.hip", "decode.hip", "prefill.hip", "indexer.hip", "attn.hip", "decode_step.hip"]
# measurement kernels for the roofline denominators (not the hot path): a library of their own
PEAK_LIB = os.path.join(HERE, "libsckv_peak.so")
PEAK_SOURCES = ["peak.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, jobs: int = 5) -> str:
    """Compile every source to an object in parallel, then link libsckv.so
    and libsckv_peak.so."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES + PEAK_SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *[f for f in FLAGS if f != "-shared"], "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and ln.strip() != ""]
        if p.returncode != 0:
            failed.append(src)
            print("\n".join(lines))
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    for lib, srcs in ((LIB, SOURCES), (PEAK_LIB, PEAK_SOURCES)):
        tmp = lib + ".tmp"
        mine = [o for o in objs if os.path.basename(o).replace(".o", ".hip") in srcs]
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *mine, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
