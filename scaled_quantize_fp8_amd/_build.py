"""Build libfp8linear.so (the FP8 linear path) and libfp8probe.so (its
measurement kernels) in-tree with hipcc for gfx950."""

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
PROBE_LIB_PATH = os.path.join(HERE, "libfp8probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "fp8l_probe.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("fp8l_device.hpp", "fp8l_quantize.hpp", "fp8l_gemm.hpp",
                                                     "fp8l_gemm3.hpp", "fp8l_gemm4.hpp", "fp8l_gemm5.hpp",
                                                     "fp8l_gemm_pair.hpp")] + [
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


def build_command(out: str = LIB_PATH, extra: list[str] | None = None,
                  sources: list[str] | None = None) -> list[str]:
    return [
        hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
        # packed fp32 VALU forms stay off (see the library's design notes)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        f'-DFP8L_SOURCE_HASH="{source_hash()}"',
        *(extra or []),
        *(SOURCES if sources is None else sources), "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Compile both libraries (always recompiles; the two hipcc runs go in
    parallel).  Returns the path of libfp8linear.so."""
    jobs = [(LIB_PATH, build_command(LIB_PATH + ".tmp")),
            (PROBE_LIB_PATH, build_command(PROBE_LIB_PATH + ".tmp", sources=PROBE_SOURCES))]
    procs = [(out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                    text=True)) for out, cmd in jobs]
    failed = []
    for out, proc in procs:
        text, _ = proc.communicate()
        msgs = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if proc.returncode != 0:
            failed.append(f"hipcc failed for {os.path.basename(out)}:\n" + "\n".join(msgs))
        elif verbose and msgs:
            print("\n".join(msgs))
    if failed:
        raise RuntimeError("\n".join(failed))
    for out, _ in jobs:
        os.replace(out + ".tmp", out)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
