"""Ahead-of-time build of libxv.so (HIP, gfx950 only).

The library is compiled in-tree with hipcc for --offload-arch=gfx950.  There is
no runtime JIT and no kernel cache: the code object in libxv.so is the only one
that ever runs.  Floating point: -ffp-contract=off, no fast-math, packed fp32
instructions disabled; every fused multiply-add is explicit in the source.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libxv.so")
SOURCES = ["xv_api.hip", "xv_gemm.hip", "xv_gdn.hip", "xv_attn.hip", "xv_greedy.hip", "xv_compose.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


def build(out: str = LIB, extra=None, verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + list(extra or []) + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature name; that warning is expected
    msgs = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed (exit %d)" % r.returncode)
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


def build_sanitized_host_checks(out_dir: str, verbose: bool = False) -> str:
    """The library's sources and a host program that calls every entry point with arguments
    breaking one of its checks (csrc/abi_sanitize_main.cpp), as one executable whose host
    code is built with AddressSanitizer and UndefinedBehaviorSanitizer (device code is
    built as usual and never runs: every call returns before any launch).  A CPU check of
    the host-side validation."""
    out = os.path.join(out_dir, "abi_sanitize")
    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(CSRC, "abi_sanitize_main.cpp")]
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-ffp-contract=off", "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include")] + srcs + ["-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout)
        raise RuntimeError("hipcc failed (exit %d)" % r.returncode)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
