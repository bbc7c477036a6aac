"""Build libsala.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m hybrid_sparse_linear_amd.build

Objects go to ``_build/`` at the repository root; the shared library is
written next to this file as ``libsala.so``.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libsala.so")

SOURCES = [
    "sala_api.cpp",
    "linear_prefill.hip",
    "linear_decode.hip",
    "neighbours.hip",
    "sparse_select.hip",
    "sparse_prefill.hip",
    "sparse_decode.hip",
    "ceilings.hip",
    "noalloc.hip",
    "sparse_backward.hip",
    "checks.hip",
]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
# Packed fp32 VALU ops stay disabled in all device code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source flags.  The sparse gradient kernels run one wave per SIMD per
# workgroup; there the compiler would keep the dK / dV accumulators in AGPRs
# and copy all 64 of them to VGPRs and back on every step (262 v_accvgpr moves
# in the loop); the VGPR form of the MFMAs keeps them in place.
PER_SOURCE = {"sparse_backward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src, verbose, build_dir, extra):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    own = PER_SOURCE.get(os.path.basename(src), [])
    cmd = ([HIPCC] + COMMON + extra + (DEVICE if src.endswith(".hip") else []) + own +
           ["-c", os.path.join(CSRC, src), "-o", obj])
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in (r.stderr or "").splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed for {src}:\n{errs}")
    if verbose and errs.strip():
        print(errs)
    return obj


def build(verbose=False, jobs=6, out=LIB, defines=()):
    """Compile every source and link the library (default: libsala.so next to this file).

    ``defines`` are extra -D flags (for building kernel variants elsewhere).
    Returns the library path.
    """
    build_dir = BUILD if out == LIB else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    extra = ["-D" + d for d in defines]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build_sanitized_abi(out_dir=None, verbose=False):
    """The C-ABI layer (sala_api.cpp, host code only) compiled with the host's
    AddressSanitizer and UndefinedBehaviorSanitizer by g++, linked with the
    kernel objects of the last build(): a library whose argument validation can
    be exercised on a machine without a GPU.  Load it with the ASan runtime
    preloaded and SALA_LIB_PATH pointing at it.  Returns its path."""
    out_dir = out_dir or os.path.join(BUILD, "sanitized")
    os.makedirs(out_dir, exist_ok=True)
    kernel_objs = [os.path.join(BUILD, os.path.basename(src) + ".o") for src in SOURCES if src != "sala_api.cpp"]
    missing = [o for o in kernel_objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"run build() first: missing {missing}")
    obj = os.path.join(out_dir, "sala_api.o")
    lib = os.path.join(out_dir, "libsala_sanitized.so")
    compile_cmd = ["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer",
                   "-fsanitize=address,undefined", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                   "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, "sala_api.cpp"), "-o", obj]
    link_cmd = ["g++", "-shared", "-o", lib, obj] + kernel_objs + ["-lasan", "-lubsan", "-L/opt/rocm/lib",
                                                                   "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    for cmd in (compile_cmd, link_cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized build failed:\n{r.stderr}")
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
