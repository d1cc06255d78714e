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
           "pa_attention_b32.hip", "pa_reduce.hip", "pa_prefill.hip"]

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


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source to an object in parallel, then link libpa.so atomically."""
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
            out, _ = p.communicate()
            # drop the expected host-side notice about the fp32-packing feature
            lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
            if lines and (verbose or p.returncode):
                print("\n".join(lines), file=sys.stderr)
            if p.returncode:
                failed.append(src)
        if failed:
            raise RuntimeError(f"hipcc failed for {failed}")
        tmp_lib = LIB + ".tmp"
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
