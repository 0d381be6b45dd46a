"""Build step of libspecdec.so: hipcc for gfx950, in-tree next to this file.

    python -m speculative_decoding_verification_specdec_amd.build
"""
from __future__ import annotations

import os
import pathlib
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
SOURCES = [PKG / "csrc" / "kernels.hip", PKG / "csrc" / "fused.hip", PKG / "csrc" / "small.hip", PKG / "csrc" / "ngram.hip",
           PKG / "csrc" / "commit.hip", PKG / "csrc" / "noalloc.hip", PKG / "csrc" / "quad.hip",
           PKG / "csrc" / "telemetry.hip", PKG / "csrc" / "api.cpp", PKG / "csrc" / "telemetry.cpp"]
HEADERS = [PKG / "csrc" / "kernels.h", PKG / "csrc" / "verify_dev.h", PKG / "csrc" / "wave_ops.h", ROOT / "include" / "specdec.h"]
OUTPUT = PKG / "libspecdec.so"
ARCH = os.environ.get("SPECDEC_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Keep the compiler from emitting packed fp32 VALU ops (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = pathlib.Path(rocm) / "bin" / "hipcc"
    return str(cand) if cand.exists() else "hipcc"


# The host code with AddressSanitizer (the device code is built as usual): for running the
# host-side checks of the C ABI under the sanitizer on a machine without a GPU.
ASAN_OUTPUT = PKG / "libspecdec_asan.so"
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
              "-Xarch_host", "-g"]


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (to preload into the process that
    loads the sanitized library)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    clang = pathlib.Path(rocm) / "llvm" / "bin" / "clang"
    res = subprocess.run([str(clang), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True)
    return res.stdout.strip()


def build_library(verbose: bool = True, asan: bool = False) -> pathlib.Path:
    out = ASAN_OUTPUT if asan else OUTPUT
    tmp = out.with_suffix(".so.tmp")
    cmd = [hipcc(), *FLAGS, *(ASAN_FLAGS if asan else []), f"-I{ROOT / 'include'}",
           *map(str, SOURCES), "-o", str(tmp)]
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"   # the host pass does not know the device feature flag
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(asan="--asan" in sys.argv[1:]))
