"""Build libpa.so in-tree with hipcc for gfx950 (cross-compiles without a GPU).

    python -m paged_kv_cache_384_amd._build
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpa.so")
SOURCES = ["pa_api.cpp", "pa_cache.hip", "pa_attention_b8.hip", "pa_attention_b16.hip",
           "pa_attention_b32.hip", "pa_reduce.hip", "pa_prefill.hip", "pa_measure.hip"]

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32 (plain fp32 VALU only).
# The host pass warns that it does not know the feature; that is expected.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]
# Per-source additions. The prefill kernel takes maxima of MFMA results; in IEEE mode each
# fmaxf operand first gets a quieting v_max_f32 x, x (64 extra VALU per key/value tile), which
# -fno-honor-nans drops. The kernel never relies on NaN propagation: slots past a context are
# zeroed by position before they reach a product.
SOURCE_FLAGS = {"pa_prefill.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


# Host-side sanitizers (AddressSanitizer, UndefinedBehaviorSanitizer) for the library's host code:
# the argument checks, planning and launch paths. Device code is compiled as usual. The library
# built with them leaves the sanitizer runtime unresolved; a process loads it first (LD_PRELOAD of
# the ASan runtime, which also carries the UBSan handlers).
HOST_SANITIZE_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                       "-Xarch_host -fno-sanitize-recover=undefined "
                       "-Xarch_host -fno-omit-frame-pointer -Xarch_host -g").split()


def asan_runtime() -> str:
    """Path of the ASan runtime shared library of hipcc's clang."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True).stdout.strip()
    return out


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    """Compile every source to an object in parallel, then link the library (libpa.so unless
    ``out`` names another path) atomically."""
    with tempfile.TemporaryDirectory(prefix="pa_build_") as tmp:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            cmd = [hipcc(), *FLAGS, *SOURCE_FLAGS.get(src, []), *extra_flags, *lang, "-c",
                   os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = []
        for src, p in procs:
            log, _ = p.communicate()
            # drop the expected host-side notice about the fp32-packing feature
            lines = [ln for ln in log.splitlines() if "packed-fp32-ops" not in ln]
            if lines and (verbose or p.returncode):
                print("\n".join(lines), file=sys.stderr)
            if p.returncode:
                failed.append(src)
        if failed:
            raise RuntimeError(f"hipcc failed for {failed}")
        tmp_lib = out + ".tmp"
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
