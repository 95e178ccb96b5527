"""Compile the gfx950 HIP library ``libmoe_mi355x.so`` in place (hipcc)."""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_mi355x.so")
SOURCES = ["api.hip", "route.hip", "route_mfma.hip", "dispatch.hip", "ffn.hip", "combine.hip",
           "backward.hip", "backward_ffn.hip", "router_backward.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # Keep packed fp32 instructions out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


# Host code only under AddressSanitizer and UndefinedBehaviorSanitizer (the
# device code is built as usual); load the result with the sanitizer runtime
# preloaded (clang's, the one hipcc links against).
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                  "-fno-omit-frame-pointer", "-shared-libsan", "-g"]


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    flags = [f for f in HIPCC_FLAGS if not (sanitize and f == "-O3")]
    if sanitize:
        flags = ["-O1", *flags, *SANITIZE_FLAGS]
    cmd = [hipcc(), *flags, "-I", os.path.join(PKG, "..", "include"), "-o", tmp, *srcs]
    res = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
