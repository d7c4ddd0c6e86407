"""Build libtsp.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

Usage: python -m long_context_transformer_amd.build [--verbose] [--resource-usage]
Every call recompiles; sources compile in parallel, then link into
long_context_transformer_amd/libtsp.so.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtsp.so")
SOURCES = ["tsp_api.hip", "tsp_gemm.hip", "tsp_attn.hip", "tsp_attn_bwd.hip", "tsp_bwd_aux.hip"]
# Per-source code generation flags. The attention kernel keeps its O accumulator and
# scores in VGPRs (MFMA "VGPR form"); the rescale of O then stays a plain VALU multiply
# instead of AGPR<->VGPR copies on every key block. It also runs with the IEEE mode bit
# off and no NaN operands assumed (its scores are finite or -inf), so max/min need no
# canonicalising moves.
SOURCE_FLAGS = {"tsp_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mno-amdgpu-ieee", "-fno-honor-nans"],
                "tsp_attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # No packed-fp32 (v_pk_*_f32) instructions anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _llvm_tool(name):
    for cand in (os.path.join("/opt/rocm/llvm/bin", name), shutil.which(name)):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError(f"{name} not found")


def check_kernel_names(obj):
    """Every kernel the host code of `obj` launches must exist under the same mangled name
    in its gfx950 code object (otherwise the launch fails at run time). The host side has a
    handle symbol per kernel, next to its __device_stub__; the device side lists kernels in
    the code object's metadata notes."""
    import tempfile
    with tempfile.TemporaryDirectory() as td:
        fatbin = os.path.join(td, "fatbin")
        code = os.path.join(td, "code")
        subprocess.run(["objcopy", f"--dump-section=.hip_fatbin={fatbin}", obj, os.path.join(td, "o")],
                       check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        subprocess.run([_llvm_tool("clang-offload-bundler"), "--unbundle", "--type=o", f"--input={fatbin}",
                        f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}", f"--output={code}"], check=True,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        notes = subprocess.run([_llvm_tool("llvm-readelf"), "--notes", code], check=True, text=True,
                               stdout=subprocess.PIPE).stdout
    device = {line.split()[1].strip("'\"") for line in notes.splitlines()
              if line.strip().startswith(".name:") and "_Z" in line}
    mangled = subprocess.run(["nm", "--defined-only", obj], check=True, text=True,
                             stdout=subprocess.PIPE).stdout.splitlines()
    demangled = subprocess.run(["nm", "-C", "--defined-only", obj], check=True, text=True,
                               stdout=subprocess.PIPE).stdout.splitlines()
    stubs = {l.split(" ", 2)[2].replace("__device_stub__", "") for l in demangled if "__device_stub__" in l}
    handles = [m.split(" ", 2)[2] for m, dm in zip(mangled, demangled)
               if dm.split(" ", 2)[1] in "dDbB" and dm.split(" ", 2)[2] in stubs]
    missing = [h for h in handles if h not in device]
    if missing or not handles:
        raise RuntimeError(f"{os.path.basename(obj)}: host kernels without a device kernel of the same "
                           f"name: {missing or 'no kernels found'}")
    return len(handles)


def build(verbose=False, resource_usage=False):
    """Compile every HIP source for gfx950 and link libtsp.so. Returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        flags = [*HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), *extra]
        out = _run([hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        return obj, out

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    for _, out in results:
        if out.strip() and (verbose or resource_usage):
            print(out)
    for obj, _ in results:
        if os.path.basename(obj) != "tsp_api.o":  # the API file launches no kernels itself
            check_kernel_names(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]], verbose)
    os.replace(tmp, LIB)
    return LIB


def device_asm(src, out_path, verbose=False):
    """gfx950 assembly of one source's device code, compiled with the library's own flags."""
    flags = [*HIPCC_FLAGS, *SOURCE_FLAGS.get(src, [])]
    _run([_hipcc(), *flags, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out_path], verbose)
    return out_path


SAN_BUILD = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(SAN_BUILD, "libtsp.so")
# Host-side sanitizers for the C ABI's host code (argument checks, workspace layout, launch
# order). Each flag applies to the host compilation only: the gfx950 code is built as usual.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]


def asan_runtime():
    """Path of the AddressSanitizer runtime that a host process must preload to use SAN_LIB."""
    out = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], check=True, text=True,
                         stdout=subprocess.PIPE, stderr=subprocess.DEVNULL).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        raise RuntimeError("AddressSanitizer runtime not found")
    return out


def build_sanitized(verbose=False):
    """libtsp.so with tsp_api.hip's host code built under AddressSanitizer and
    UndefinedBehaviorSanitizer (the other objects as in `build`, which must have run).
    Returns the library path."""
    hipcc = _hipcc()
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "tsp_api.hip"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"run build() first: {missing}")
    os.makedirs(SAN_BUILD, exist_ok=True)
    api = os.path.join(SAN_BUILD, "tsp_api.o")
    _run([hipcc, *HIPCC_FLAGS, *SAN_FLAGS, "-c", os.path.join(CSRC, "tsp_api.hip"), "-o", api], verbose)
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", SAN_LIB, api, *objs], verbose)
    return SAN_LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    ap.add_argument("--sanitize", action="store_true",
                    help="also build the host-sanitized library (ASan + UBSan) under _build_san/")
    args = ap.parse_args(argv)
    path = build(verbose=args.verbose, resource_usage=args.resource_usage)
    print(path)
    if args.sanitize:
        print(build_sanitized(verbose=args.verbose))


if __name__ == "__main__":
    sys.exit(main())
