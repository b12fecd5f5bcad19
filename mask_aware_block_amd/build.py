"""Build libfmask.so (HIP, gfx950) in-tree with hipcc.

Every .hip file under csrc/ is compiled for gfx950 and linked into
mask_aware_block_amd/libfmask.so.  Packed FP32 VALU instructions are disabled
for the device pass (-packed-fp32-ops); hipcc's host pass warns that it does
not know that feature, which is harmless.
"""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfmask.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]

# Per-source additions.  attn_bwd.hip: its dK/dV kernel runs one wave per SIMD
# with more than 256 registers live; left to its heuristics the compiler gives
# every MFMA of that kernel accumulator-register (AGPR) operands and then
# copies the scores to VGPRs for the VALU and the gradients back and forth
# (about 700 v_accvgpr moves per launch of the loop body).  VGPR-form MFMAs
# leave 44 such moves and run the backward about 5% faster, bit-identically.
PER_FILE = {
    "attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, extra):
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *PER_FILE.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(extra=(), verbose=False):
    """Compile every HIP source and link libfmask.so; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host-only build for the sanitizers: the host side of every source (argument
# checks, size arithmetic, descriptor validation) under AddressSanitizer and
# UndefinedBehaviorSanitizer, with no device code at all, so that it loads and
# runs where there is no GPU.  Each -fsanitize= applies to the host pass only.
# Each object embeds an empty GPU binary where the device pass would put the
# kernels' code object, so the library links and loads with no kernel in it.
SANITIZE_HOST = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
]
CLANGXX = os.environ.get("CLANGXX", "/opt/rocm/llvm/bin/clang++")


def build_host_sanitized(outdir):
    """Compile the host side of every source with ASan and UBSan into
    outdir/libfmask_host_san.so (no device code); returns its path."""
    os.makedirs(outdir, exist_ok=True)
    empty = os.path.join(outdir, "no_kernels.bin")
    open(empty, "wb").close()

    def comp(src):
        obj = os.path.join(outdir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, "--offload-host-only", "-Xclang", "-fcuda-include-gpubinary", "-Xclang", empty,
               *SANITIZE_HOST, "-g", "-O1", "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"host-only compile failed on {src}:\n{r.stderr}")
        return obj

    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(comp, srcs))
    lib = os.path.join(outdir, "libfmask_host_san.so")
    # (host objects only: linked by the host compiler with the sanitizer runtimes)
    link = [CLANGXX, "-shared", "-fsanitize=address,undefined", *objs, "-L/opt/rocm/lib", "-lamdhip64",
            "-Wl,-rpath,/opt/rocm/lib", "-o", lib]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return lib


if __name__ == "__main__":
    build(extra=sys.argv[1:], verbose=True)
