"""Build the HIP library (gfx950) in-tree: bidirectional_lstm_sequence_amd/libbilstm_amd.so."""

from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libbilstm_amd.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
OBJ_DIR = os.path.join(PKG, "_build")

SOURCES = ["host_plan.cpp", "host_pack_schedule.cpp", "host_heads.cpp", "host_library_projection.cpp",
           "kernels_projection.hip", "kernels_recurrence.hip", "kernels_heads.hip",
           "forward_noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument",
    # packed FP32 VALU ops stay off: the compiler would otherwise form v_pk_* from float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library. Always rebuilds."""
    os.makedirs(OBJ_DIR, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
        if verbose and res.stderr.strip():
            print(res.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    # hipBLASLt: the vendor-GEMM projection offered as a comparator (bilstm_options.projection)
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
           "-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


MODEL_SOURCE = os.path.join(CSRC, "protocol_model.cpp")
MODEL_LIB = os.path.join(PKG, "libbilstm_protocol_model.so")


def build_protocol_model(out_path: str = MODEL_LIB, source_dir: str = CSRC, extra=(), main: bool = False) -> str:
    """Compile the CPU model of the publication protocols (host only, g++).

    ``source_dir`` holds protocol_model.cpp and the protocol.h it includes (the tests compile
    copies with planted mistakes); ``main`` builds the stand-alone driver executable instead of
    the shared library; ``extra`` adds flags (e.g. ``-fsanitize=thread``)."""
    src = os.path.join(source_dir, "protocol_model.cpp")
    kind = ["-DBILSTM_MODEL_MAIN"] if main else ["-shared", "-fPIC"]
    tmp = out_path + ".tmp"
    cmd = ["g++", "-O2", "-g", "-std=c++17", "-pthread", "-Wall", "-Wextra", *kind, *extra,
           "-I", source_dir, src, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"g++ failed for the protocol model:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_protocol_model())
