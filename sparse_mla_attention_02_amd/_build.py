"""Build the HIP library ``libsmla.so`` in-tree for gfx950 with hipcc."""

from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsmla.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
          # keep the compiler from forming packed fp32 VALU instructions
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]
KERNELS = os.path.join(CSRC, "smla_kernels.hip")
HOST = os.path.join(CSRC, "smla_host.cpp")
EXAMPLE_SRC = os.path.join(CSRC, "example", "smla_example.cpp")
EXAMPLE = os.path.join(PKG, "smla_example")


def commands(out: str, tmp: str) -> list:
    """The compile and link commands: the kernel file twice (the pipelined and
    general kernels with MFMA results in VGPRs, so that the pipelined kernel's
    epilogue reads its scores without a copy; the softmax_lse kernel with the
    compiler's default), the host code once, then one shared library."""
    main_o = os.path.join(tmp, "kernels.o")
    lse_o = os.path.join(tmp, "kernels_lse.o")
    host_o = os.path.join(tmp, "host.o")
    cc = hipcc()
    return [
        [cc, *COMMON, "-mllvm", "-amdgpu-mfma-vgpr-form", "-x", "hip", "-c", KERNELS, "-o", main_o],
        [cc, *COMMON, "-DSMLA_LSE_TU", "-x", "hip", "-c", KERNELS, "-o", lse_o],
        [cc, *COMMON, "-x", "hip", "-c", HOST, "-o", host_o],
        [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", main_o, lse_o, host_o, "-o", out],
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msg)
    if verbose and msg.strip():
        print(msg, flush=True)


def example_command(out: str) -> list:
    """The example host program on the C ABI, linked against libsmla.so in
    the same folder."""
    return [hipcc(), "-O2", "-std=c++17", "-Wall", "-I", INCLUDE, EXAMPLE_SRC, "-L", PKG,
            "-lsmla", "-Wl,-rpath,$ORIGIN", "-o", out]


def build(verbose: bool = False) -> str:
    """Compile every source into ``libsmla.so`` and the example program
    (always recompiles)."""
    import tempfile
    out = LIB + ".tmp%d" % os.getpid()
    with tempfile.TemporaryDirectory(prefix="smla_build_") as tmp:
        for cmd in commands(out, tmp):
            _run(cmd, verbose)
    os.replace(out, LIB)
    exe = EXAMPLE + ".tmp%d" % os.getpid()
    _run(example_command(exe), verbose)
    os.replace(exe, EXAMPLE)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
