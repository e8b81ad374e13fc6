"""Sanitizer builds of the host-side code (CPU only; the tests in tests/test_sanitizers.py run them).

* the library's host code under AddressSanitizer and UndefinedBehaviorSanitizer: every source
  of the library compiled as for the product, with the sanitizers on the host side only (the
  GPU code is built as usual), linked with host_check_main.cpp into an executable that runs the
  packer, the schedule and every entry point's argument checks;
* the CPU model of the publication protocols under ThreadSanitizer (protocol_model.cpp's
  stand-alone driver).

The oracle's own sanitizer build is in oracle/__init__.py (build_check).
"""

from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

from . import _build

HOST_SANITIZERS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-sanitize-recover=all"]


def build_host_check(out_dir: str) -> str:
    """Compile the library's sources and host_check_main.cpp with host-side ASan + UBSan."""
    os.makedirs(out_dir, exist_ok=True)
    flags = [f"--offload-arch={_build.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(_build.ROOT, "include"), *HOST_SANITIZERS]

    def compile_one(src: str) -> str:
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        cmd = [_build.HIPCC, *flags, "-x", "hip", "-c", os.path.join(_build.CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as pool:
        objs = list(pool.map(compile_one, [*_build.SOURCES, "host_check_main.cpp"]))
    exe = os.path.join(out_dir, "host_check")
    cmd = [_build.HIPCC, f"--offload-arch={_build.ARCH}", *HOST_SANITIZERS, *objs, "-L/opt/rocm/lib",
           "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    return exe


def build_protocol_model_tsan(out_dir: str) -> str:
    """The protocol model's stand-alone driver under ThreadSanitizer (g++, host only)."""
    os.makedirs(out_dir, exist_ok=True)
    return _build.build_protocol_model(os.path.join(out_dir, "protocol_model_tsan"), main=True,
                                       extra=["-fsanitize=thread"])
