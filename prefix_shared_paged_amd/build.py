"""Build libsgl_attn.so (HIP kernels for gfx950 + host bookkeeping + C ABI) in-tree.

    python -m prefix_shared_paged_amd.build [-v]

Every source is compiled with hipcc for gfx950 only; packed-fp32 instructions
are disabled for the device code (-Xclang -target-feature -Xclang
-packed-fp32-ops).  Objects go to prefix_shared_paged_amd/_build/, the library
to prefix_shared_paged_amd/libsgl_attn.so.
"""
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsgl_attn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["host_cache.cpp", "api.hip", "kernels_misc.hip", "kernels_f32.hip",
           "kernels_decode.hip", "kernels_decode_rows.hip", "kernels_mla.hip", "kernels_extend.hip",
           "kernels_hicache.hip", "kernels_probe.hip"]

FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + INCLUDE, "-I" + CSRC]

# Per-source flags.  The decode kernel keeps its MFMA accumulators in ordinary
# VGPRs: its softmax rescales them with vector ALU ops, and AGPR accumulators
# would be copied to VGPRs and back around every such rescale, costing both
# instructions and the registers that decide how many waves fit per CU.
# The extend kernel is built without NaN semantics: its row maxima then take
# the MFMA results straight into v_max3 (with NaNs honoured every such chain
# first copies its inputs through a quieting v_max), four VALU ops per tile
# fewer.  Its inputs are finite by contract; infinities (the causal mask's
# -inf) keep their meaning.
SOURCE_FLAGS = {"kernels_extend.hip": ["-fno-honor-nans"],
                "kernels_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
                "kernels_decode_rows.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
                "kernels_mla.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def _compile(src, verbose):
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + SOURCE_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", out]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-x", "hip"] + cmd[1:]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so: harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs))
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
