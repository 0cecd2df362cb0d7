"""Build libattn.so (the C-ABI HIP library) in-tree with hipcc for gfx950.

Usage: python -m attention_forward_02_amd.build [-v]

Each source compiles to its own object (in parallel), then hipcc links the
shared library.  The kernels of each head dimension are a translation unit
of their own so that each gets the register-form options that suit it.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
# Standalone probe of the chip's MFMA and VALU ceilings (not part of the library).
CEILING = os.path.join(PKG, "chip_ceiling")
# Timeline probe: two kernels with their shader-clock trace points, a library
# of its own (attn_timeline.hip, read by timeline.py).
TIMELINE_LIB = os.path.join(PKG, "libattn_timeline.so")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Packed FP32 VALU forms stay off: hipcc would otherwise emit them from
    # ordinary float2 arithmetic.  The host pass ignores the flag.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # No NaN-quieting copies around fmaxf in the row-max reductions.
    "-fno-honor-nans",
]
# MFMA accumulators in ordinary VGPRs: the softmax reads and rescales them
# every tile, and AGPR-resident accumulators would need copies.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
# The scheduler's AMDGPU register-pressure trackers: at 16-bit d = 128 they
# fit the pipelined kernel in 254 VGPRs without the 36-byte scratch spill of
# the default tracker (same speed; no spill traffic).
TRACKERS = ["-mllvm", "-amdgpu-use-amdgpu-trackers=1"]

SOURCES = [
    ("attn_api.cpp", []),
    ("attn_dispatch.cpp", []),
    ("attn_fwd_d64.hip", VGPR_FORM),
    ("attn_fwd_d128.hip", VGPR_FORM + TRACKERS),
    # 64 rows per wave, one wave per SIMD: the default (AGPR) form keeps the
    # output accumulators in AGPRs.
    ("attn_fwd_d128_wide.hip", []),
    # tile-size variants: the 128-key bf16 kernel spills under the trackers
    ("attn_fwd_d128_bc.hip", VGPR_FORM),
    ("attn_fwd_d256.hip", VGPR_FORM),
    ("attn_fwd_d64_fp8.hip", VGPR_FORM),
    ("attn_fwd_d128_fp8.hip", VGPR_FORM),
    ("attn_fwd_d256_fp8.hip", VGPR_FORM),
    ("attn_fwd_splitkv.hip", VGPR_FORM),
    ("attn_quant.hip", []),
]
# The timeline probe's two builds of attn_timeline.hip, each with the options
# of the library unit that holds its kernel.
TIMELINE_SOURCES = [
    ("attn_timeline.hip", VGPR_FORM + ["-DATTN_TIMELINE_KERNEL=0"], "attn_timeline_seq.o"),
    ("attn_timeline.hip", VGPR_FORM + TRACKERS + ["-DATTN_TIMELINE_KERNEL=1"], "attn_timeline_producer.o"),
]


def hipcc():
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; set ROCM_PATH")


def compile_command(src, extra, obj):
    return [hipcc(), *COMMON, *extra, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {' '.join(cmd)}")
    return res


def build(verbose=False):
    """Compile every source and link libattn.so next to this file (always
    recompiles) and return its path."""
    with tempfile.TemporaryDirectory(prefix="attn_build_") as tmp:
        objs, cmds = [], []
        for src, extra in SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            objs.append(obj)
            cmds.append(compile_command(src, extra, obj))
        tl_objs = [os.path.join(tmp, name) for _, _, name in TIMELINE_SOURCES]
        cmds += [compile_command(src, extra, obj) for (src, extra, _), obj in zip(TIMELINE_SOURCES, tl_objs)]
        workers = min(len(cmds), max(1, (os.cpu_count() or 2)))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        out = LIB + ".tmp"
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out], verbose)
        os.replace(out, LIB)
        out = TIMELINE_LIB + ".tmp"
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *tl_objs, "-o", out], verbose)
        os.replace(out, TIMELINE_LIB)
        exe = os.path.join(tmp, "chip_ceiling")
        _run([hipcc(), *[f for f in COMMON if f != "-fPIC"], os.path.join(CSRC, "chip_ceiling.hip"), "-o", exe], verbose)
        shutil.move(exe, CEILING)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
