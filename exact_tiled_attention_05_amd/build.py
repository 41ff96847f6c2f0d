"""Build libfa.so (the C-ABI attention library) in-tree with hipcc for gfx950.

Usage: ``python -m exact_tiled_attention_05_amd.build [--all]`` or ``build()`` / ``build_all()``
from Python (``--all`` / ``build_all`` also build the race-check library). The library
lands next to this file, where the Python binding loads it from. Each translation unit is compiled
to an object with its own flags, then the objects are linked into one shared library.
"""
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")
# The same sources built with FA_RACE_CHECK=1: every LDS tile load completes before any wave goes
# on and LDS starts filled with NaN (see fa_device.h); the tests compare it with libfa.so bit for
# bit.
RACE_CHECK_LIB_PATH = os.path.join(PKG_DIR, "libfa_race.so")

# Packed fp32 VALU instructions are disabled for all device code. NaNs are never produced by the
# kernels for finite inputs (hidden keys are -inf, never 0*inf), so max needs no NaN handling.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-honor-nans",
    "-Wall", "-Wno-unused-result",
]

# Translation units of the library and the extra flags of each. The wide-row forward kernel needs
# about 360 registers per lane; with its MFMA results forced into VGPRs the Q operands go to AGPRs
# (read directly by the MFMAs) instead of the accumulators the softmax reads and rescales. The
# flag is kept to that file so that it changes no other kernel. The wide dK/dV kernel of the
# backward pass has its own file too: it keeps the compiler's default form (its accumulators in
# AGPRs) and writes out the MFMAs whose results belong in VGPRs.
SOURCES = [
    ("fa_api.hip", []),
    ("fa_wide.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"]),
    ("fa_bwd_wide.hip", []),
]


def hipcc_path():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only feature flag; that warning is harmless.
    msgs = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (r.returncode, "\n".join(msgs)))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)


def build(verbose=False, extra_flags=(), out=LIB_PATH):
    """Compile the library's translation units and link them into ``out``; returns its path."""
    tag = "%d" % os.getpid()
    objs = []
    try:
        for src, flags in SOURCES:
            obj = os.path.join(os.path.dirname(out), "%s.%s.o" % (os.path.splitext(src)[0], tag))
            _run([hipcc_path()] + HIP_FLAGS + flags + list(extra_flags) +
                 ["-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        tmp = out + ".tmp" + tag
        _run([hipcc_path(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp],
             verbose)
        os.replace(tmp, out)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return out


def build_all(verbose=False):
    """Build libfa.so and its race-check twin libfa_race.so."""
    build(verbose=verbose)
    build(verbose=verbose, extra_flags=["-DFA_RACE_CHECK=1"], out=RACE_CHECK_LIB_PATH)


if __name__ == "__main__":
    if "--all" in sys.argv:
        build_all(verbose="-v" in sys.argv)
        print(LIB_PATH, RACE_CHECK_LIB_PATH)
    else:
        print(build(verbose="-v" in sys.argv))
