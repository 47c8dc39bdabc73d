"""Build libegm.so (the C-ABI library) in-tree with hipcc for gfx950.

    python dense_gemm_epilogue_fp16_amd/build.py      # or build() from Python (loads this file by path)

Translation units: egm_kernels.hip once per 16-bit dtype (fp16, bf16) and
once per (fp8 format pair, output dtype), and the host API egm_api.hip,
compiled in parallel (objects under _build/), then linked into one shared
library next to this file.

    python dense_gemm_epilogue_fp16_amd/build.py --host-sanitized

builds _build/libegm_host_sanitized.so: the same kernels, with the host API
unit compiled under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only: each -fsanitize= goes behind -Xarch_host, so no device code is
instrumented).  It is for CPU runs of the ABI tests, with the sanitizer
runtime preloaded into the Python process (see host_sanitizer_runtime()).
"""
from __future__ import annotations

import os
import glob
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libegm.so")
PROBE_LIB = os.path.join(HERE, "libegm_probe.so")  # the MFMA-shape power probe (benchmark only)
OBJ_DIR = os.path.join(HERE, "_build")
SANITIZED_LIB = os.path.join(OBJ_DIR, "libegm_host_sanitized.so")
ARCH = "gfx950"

# Packed fp32 ops (v_pk_*_f32) are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-Wall",
          "-Wno-unused-command-line-argument"]
# host-side sanitizers for the host API unit (never applied to device code)
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _units(obj_dir: str):
    kernels = os.path.join(CSRC, "egm_kernels.hip")
    units = [
        (kernels, os.path.join(obj_dir, "egm_kernels_f16.o"), ["-DEGM_DTYPE=0"]),
        (kernels, os.path.join(obj_dir, "egm_kernels_bf16.o"), ["-DEGM_DTYPE=1"]),
        (os.path.join(CSRC, "egm_api.hip"), os.path.join(obj_dir, "egm_api.o"), []),
    ]
    # the lean 256x256 tile (16x16x32 blocks, one set of A fragments): its
    # kernels only, in units whose instruction scheduler keeps them free of
    # scratch (the default scheduler spills all of them): the ILP-first
    # scheduler for B not transposed with the forward epilogues (3-4 % faster
    # than the register-minimising one there), the register-minimising
    # scheduler for the rest (the ILP-first one spills those).  The other
    # kernels keep the default, under which they measured fastest.
    for dt, name in ((0, "f16"), (1, "bf16")):
        units.append((kernels, os.path.join(obj_dir, f"egm_kernels_lean1_{name}.o"),
                      [f"-DEGM_DTYPE={dt}", "-DEGM_LEAN=1", "-mllvm", "-amdgpu-sched-strategy=max-ilp"]))
        units.append((kernels, os.path.join(obj_dir, f"egm_kernels_lean2_{name}.o"),
                      [f"-DEGM_DTYPE={dt}", "-DEGM_LEAN=2", "-mllvm", "-amdgpu-sched-strategy=iterative-minreg"]))
    # fp8 operands: one unit per (output dtype, format pair)
    for dt in (0, 1):
        for f8 in (1, 2, 3, 4):
            units.append((kernels, os.path.join(obj_dir, f"egm_kernels_fp8_{dt}_{f8}.o"),
                          [f"-DEGM_DTYPE={dt}", f"-DEGM_F8={f8}"]))
    return units


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every HIP translation unit for gfx950 and link libegm.so."""
    cc = hipcc()
    extra = list(extra_flags or [])
    os.makedirs(OBJ_DIR, exist_ok=True)
    units = _units(OBJ_DIR)
    cmds = [[cc, *COMMON, *DEVICE_FLAGS, *defs, *extra, "-c", src, "-o", obj] for src, obj, defs in units]
    with ThreadPoolExecutor(min(len(cmds), max(1, os.cpu_count() or 1))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for _, o, _ in units]], verbose)
    os.replace(tmp, LIB)
    # the measurement probe: a library of its own, loaded only by bench.py --mfma-shape-probe
    tmp = PROBE_LIB + ".tmp"
    _run([cc, *COMMON, *DEVICE_FLAGS, "-shared", os.path.join(CSRC, "egm_mfma_probe.hip"), "-o", tmp], verbose)
    os.replace(tmp, PROBE_LIB)
    return LIB


def host_sanitizer_runtime() -> str:
    """Path of clang's AddressSanitizer runtime (it carries the
    UndefinedBehaviorSanitizer handlers too), to preload into the process
    that loads the sanitized library."""
    cc = os.path.realpath(hipcc())
    roots = [os.path.join(os.path.dirname(os.path.dirname(cc)), "llvm"), "/opt/rocm/llvm",
             os.path.dirname(os.path.dirname(cc))]
    for root in roots:
        hits = sorted(glob.glob(os.path.join(root, "lib", "clang", "*", "lib", "linux",
                                             "libclang_rt.asan-x86_64.so")))
        if hits:
            return hits[-1]
    raise RuntimeError("clang's AddressSanitizer runtime (libclang_rt.asan-x86_64.so) not found")


def build_host_sanitized(verbose: bool = False) -> str:
    """The library with its host API unit under ASan + UBSan (host code only)
    and the kernel objects of the last build(); builds those first if absent."""
    cc = hipcc()
    units = _units(OBJ_DIR)
    kernel_objs = [o for src, o, _ in units if not src.endswith("egm_api.hip")]
    if not all(os.path.exists(o) for o in kernel_objs):
        build(verbose)
    api_src = os.path.join(CSRC, "egm_api.hip")
    api_obj = os.path.join(OBJ_DIR, "egm_api_host_sanitized.o")
    _run([cc, *COMMON, *DEVICE_FLAGS, *HOST_SANITIZE, "-c", api_src, "-o", api_obj], verbose)
    tmp = SANITIZED_LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", tmp, api_obj, *kernel_objs], verbose)
    os.replace(tmp, SANITIZED_LIB)
    return SANITIZED_LIB


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
