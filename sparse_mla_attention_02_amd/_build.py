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
# (source, extra hipcc flags): the pipelined and general kernels keep MFMA
# results in VGPRs (-amdgpu-mfma-vgpr-form), so that their epilogues read the
# scores without a copy; the softmax_lse kernel, with one 32-head block per
# wave, is faster with the compiler's default
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
SOURCES = [
    ("smla_wide.hip", VGPR_FORM),
    ("smla_narrow.hip", VGPR_FORM),
    ("smla_general.hip", VGPR_FORM),
    ("smla_lse_wide.hip", VGPR_FORM),
    ("smla_lse.hip", []),
    ("smla_dispatch.cpp", []),
    ("smla_host.cpp", []),
]
# Kernels laid out to keep every value in registers: the build fails if the
# compiler gives any of them scratch memory (a spill there would put memory
# waits into the MFMA pipeline without any other sign). The general kernel's
# 128-head variants without the staged row keep two registers in scratch.
NO_SCRATCH = {"smla_wide.hip", "smla_narrow.hip", "smla_lse_wide.hip", "smla_lse.hip"}
RESOURCE_REMARKS = ["-Rpass-analysis=kernel-resource-usage"]
# the source files of each kernel (its own file and the shared device code)
KERNEL_SOURCES = {
    "smla_wide_kernel": ("smla_wide.hip", "smla_device.h", "smla_internal.h"),
    "smla_narrow_kernel": ("smla_narrow.hip", "smla_device.h", "smla_internal.h"),
    "smla_l1norm_kernel": ("smla_general.hip", "smla_device.h", "smla_internal.h"),
    "smla_lse_kernel": ("smla_lse.hip", "smla_device.h", "smla_internal.h"),
    "smla_lse_wide_kernel": ("smla_lse_wide.hip", "smla_device.h", "smla_internal.h"),
    "smla_lse_narrow_kernel": ("smla_narrow.hip", "smla_device.h", "smla_internal.h"),
}
EXAMPLE_SRC = os.path.join(CSRC, "example", "smla_example.cpp")
EXAMPLE = os.path.join(PKG, "smla_example")


def kernel_source_sha256(kernel: str) -> str:
    """sha256 over the source files of one kernel, in a fixed order."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def commands(out: str, tmp: str) -> tuple:
    """The compile commands (independent of each other) and the link
    command of the shared library."""
    cc = hipcc()
    compiles, objs = [], []
    for src, extra in SOURCES:
        obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
        remarks = RESOURCE_REMARKS if src in NO_SCRATCH else []
        compiles.append([cc, *COMMON, *extra, *remarks, "-x", "hip", "-c",
                         os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    link = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", out]
    return compiles, link


def scratch_users(text: str) -> list:
    """(kernel, bytes per lane) of every kernel with scratch memory, from
    the compiler's kernel-resource-usage remarks."""
    out, name = [], None
    for line in text.splitlines():
        if "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].strip()
        if body.startswith("Function Name:"):
            name = body.split(":", 1)[1].split()[0]
        elif body.startswith("ScratchSize [bytes/lane]:"):
            n = int(body.split(":", 1)[1].split()[0])
            if n:
                out.append((name, n))
    return out


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    lines = (res.stdout + res.stderr).splitlines()
    msg = "\n".join(l for l in lines
                    if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msg)
    if RESOURCE_REMARKS[0] in cmd:
        spills = scratch_users("\n".join(lines))
        if spills:
            raise RuntimeError("kernels that must not use scratch memory do: " +
                               ", ".join(f"{k} ({n} bytes per lane)" for k, n in spills))
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
    from concurrent.futures import ThreadPoolExecutor
    with tempfile.TemporaryDirectory(prefix="smla_build_") as tmp:
        compiles, link = commands(out, tmp)
        with ThreadPoolExecutor(max_workers=min(len(compiles), os.cpu_count() or 1)) as ex:
            for f in [ex.submit(_run, c, verbose) for c in compiles]:
                f.result()
        _run(link, verbose)
    os.replace(out, LIB)
    exe = EXAMPLE + ".tmp%d" % os.getpid()
    _run(example_command(exe), verbose)
    os.replace(exe, EXAMPLE)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
