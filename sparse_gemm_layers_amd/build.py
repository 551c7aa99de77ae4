"""Builds libsg.so (the C-ABI library) for gfx950 with hipcc, in place.

Usage: python -m sparse_gemm_layers_amd.build   (or __graft_entry__.build()).
Every .hip file under csrc/ is compiled to an object in parallel, then linked
into sparse_gemm_layers_amd/libsg.so.

python -m sparse_gemm_layers_amd.build --host-sanitizers builds a second copy,
_build/san/libsg_hostsan.so, whose HOST code (argument checks, launch set-up)
is instrumented with AddressSanitizer and UndefinedBehaviorSanitizer; device
code is built as usual and not instrumented.  Load it with the sanitizer
runtime preloaded (HOST_SANITIZER_RUNTIME) and SG_LIBRARY pointing at it; the
CPU-only ABI tests run that way (tests/test_abi_sanitized.py).
"""
import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsg.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # no packed fp32 arithmetic anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in VGPRs: the promotion FMAs read them directly
    # instead of copying them out of AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


# Per-source extra flags.  The FP8 GEMM / decode kernels schedule better with
# the ILP-maximising machine scheduler (decode 1-4% faster on MI355X, the
# large-M kernels unchanged); the quantisers and the weight-only kernels were
# slower with it, so the library as a whole keeps the default.
SRC_FLAGS = {"gemm_fp8.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


# Host-only sanitizers: each -fsanitize= applies to the host pass alone.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]
SAN_DIR = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_DIR, "libsg_hostsan.so")


def host_sanitizer_runtime() -> str:
    """Path of the shared AddressSanitizer runtime that must be preloaded into an
    uninstrumented process (python) before it loads the sanitized library."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def _compile(src: str, sanitize: bool = False) -> str:
    out_dir = SAN_DIR if sanitize else BUILD
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    extra = SAN_FLAGS + ["-O1"] if sanitize else SRC_FLAGS.get(os.path.basename(src), [])
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in r.stderr.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = True, sanitize: bool = False) -> str:
    out_dir, lib = (SAN_DIR, SAN_LIB) if sanitize else (BUILD, LIB)
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, sanitize), srcs))
    tmp = lib + ".tmp"
    link_extra = ["-shared-libsan", *SAN_FLAGS] if sanitize else []
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources")
    return lib


if __name__ == "__main__":
    build(sanitize="--host-sanitizers" in sys.argv[1:])
