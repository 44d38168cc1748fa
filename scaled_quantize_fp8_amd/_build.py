"""Build libfp8linear.so in-tree with hipcc for gfx950."""

from __future__ import annotations

import hashlib
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libfp8linear.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = [os.path.join(CSRC, "fp8l_api.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("fp8l_device.hpp", "fp8l_quantize.hpp", "fp8l_gemm.hpp",
                                                     "fp8l_gemm3.hpp", "fp8l_gemm4.hpp", "fp8l_gemm5.hpp")] + [
    os.path.join(ROOT, "include", "fp8linear.h")
]


def source_hash() -> str:
    """SHA-256 over the library's sources and its public header (file names
    and bytes, in sorted order).  The build compiles it into the library
    (fp8_source_hash), so a library built from other sources is detected."""
    h = hashlib.sha256()
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                   if f.endswith((".hip", ".hpp", ".h")))
    files.append(os.path.join(ROOT, "include", "fp8linear.h"))
    for path in files:
        h.update(os.path.relpath(path, ROOT).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build_command(out: str = LIB_PATH, extra: list[str] | None = None) -> list[str]:
    return [
        hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
        # packed fp32 VALU forms stay off (see the library's design notes)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        f'-DFP8L_SOURCE_HASH="{source_hash()}"',
        *(extra or []),
        *SOURCES, "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Compile the HIP library; always recompiles.  Returns the .so path."""
    tmp = LIB_PATH + ".tmp"
    cmd = build_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
