"""Build the HIP library libfp.so in-tree for gfx950 (hipcc, no JIT cache)."""

from __future__ import annotations

import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libfp.so")
SOURCES = [os.path.join(HERE, "csrc", "fp_lib.hip")]
# measurement microbenchmarks (read stream, MFMA loop), a library of their own
PEAKS_LIB = os.path.join(HERE, "libfp_peaks.so")
PEAKS_SOURCES = [os.path.join(HERE, "csrc", "fp_peaks.hip")]
DEPS = SOURCES + [os.path.join(HERE, "csrc", f) for f in ("fp_kernels.h", "fp_device.h", "fp_decode.h", "fp_prefill.h",
                                                                "fp_stats.h", "fp_lora.h", "fp_evict.h")] + [
    os.path.join(ROOT, "include", "fp.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs rather than AGPRs: the attention-mass kernel reads
    # every score with VALU instructions, which cannot take AGPR operands, so
    # AGPR results would cost one copy per score (the attention kernels are
    # unchanged by it)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


# The host code (validation, planning, accounting, frame merging) built with
# AddressSanitizer and UndefinedBehaviorSanitizer for the CPU tests; device
# code is compiled as usual and never instrumented.
ASAN_LIB = os.path.join(HERE, "libfp_hostsan.so")
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def source_hash(paths=None) -> str:
    """SHA-256 over the library's source files (DEPS, in order), as compiled into fp_source_hash()."""
    h = hashlib.sha256()
    for p in (DEPS if paths is None else paths):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + b"\0" + f.read())
    return h.hexdigest()


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile libfp.so (always recompiles). Returns the library path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra_flags or []) + [f'-DFP_SOURCE_HASH="{source_hash()}"',
                                                               "-I", os.path.join(ROOT, "include")] + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libfp.so")
    os.replace(tmp, LIB)
    ptmp = PEAKS_LIB + ".tmp"
    pcmd = [hipcc()] + HIPCC_FLAGS + PEAKS_SOURCES + ["-o", ptmp]
    if verbose:
        print(" ".join(pcmd), flush=True)
    res = subprocess.run(pcmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libfp_peaks.so")
    os.replace(ptmp, PEAKS_LIB)
    return LIB




def build_host_sanitized(verbose: bool = False) -> str:
    """Compile libfp_hostsan.so: libfp.so with its host code under ASan + UBSan."""
    tmp = ASAN_LIB + ".tmp"
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O1"]
    cmd = [hipcc()] + flags + SANITIZE_FLAGS + [f'-DFP_SOURCE_HASH="{source_hash()}"',
                                                "-I", os.path.join(ROOT, "include")] + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libfp_hostsan.so")
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


def sanitizer_runtime() -> str:
    """Path of the clang AddressSanitizer runtime (preloaded into the process that loads libfp_hostsan.so)."""
    res = subprocess.run([os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang"),
                          "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang's AddressSanitizer runtime was not found")
    return path


if __name__ == "__main__":
    print(build(verbose=True))
